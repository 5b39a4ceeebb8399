// Host-side schedule builder: per-CU instruction queues and the packed-weight
// stream layout.  Pure C++ (no HIP), so it also runs on machines without a GPU.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_internal.h"

namespace mk {

// Source matrices of the pack table.  Layer matrices: layer * MATS_PER_LAYER + kind.
enum MatKind : uint32_t { MAT_WQ = 0, MAT_WK, MAT_WV, MAT_WO, MAT_GATE, MAT_UP, MAT_DOWN, MATS_PER_LAYER };

// One row of one stream: copy src[row][k0 .. k0+klen) (bf16), zero-pad to kunits*512.
struct PackRow {
    uint32_t mat;
    uint32_t row;
    uint32_t k0;
    uint32_t klen;
    uint32_t src_cols;   // row length of the source matrix
    uint32_t kunits;
    uint32_t ustride;    // stream units from one of the row's units to the next (2: interleaved with
                         // the other row of its row-group)
    uint32_t reserved;
    uint64_t dst_unit;   // absolute unit index in the packed buffer (first unit; later units every
                         // ustride * NW)
};

struct Plan {
    // shape
    int L = 0, H = 0, Hq = 0, Hkv = 0, D = 0, F = 0, V = 0, B = 0, max_seq = 0, G = 0;
    bool tied = true;
    float eps = 0, theta = 0;
    // schedule parameters
    int ncu = 0, n_split = 0, n_chunk = 0;
    int ku_h = 0, ku_q = 0, ku_f = 0;
    int chunk_begin[17] = {0};
    int n_stages = 0;
    // queues
    std::vector<Inst> insts;             // queues back to back
    std::vector<uint32_t> queue_begin;   // [ncu + 1]
    std::vector<uint32_t> stage_pc;      // [ncu * (n_stages + 1)]
    std::vector<uint32_t> unit_off;      // [(queue_begin[cu] + cu + pc) * NW + w]
    // streams
    std::vector<uint64_t> stream_base;   // [ncu * NW] unit 0 of each stream; unit k at base + k * NW
    std::vector<uint64_t> stream_len;    // [ncu * NW]
    uint64_t total_units = 0;
    std::vector<PackRow> pack;

    int lm_mat() const { return L * MATS_PER_LAYER; }
    int n_mats() const { return L * MATS_PER_LAYER + 1; }
};

// Checks the config against the kernels' limits; fills `err` on failure.
int validate_config(const mk_config& cfg, std::string& err);

// Builds the queues and stream layout for `ncu` workgroups.
int build_plan(const mk_config& cfg, int ncu, Plan& out, std::string& err);

// Checks that every output is produced exactly once per step and simulates the
// queues (each instruction runs once everything it reads has been produced);
// returns false with a message on a coverage hole, a duplicate or a deadlock.
bool check_plan(const Plan& p, std::string& err);

}  // namespace mk
