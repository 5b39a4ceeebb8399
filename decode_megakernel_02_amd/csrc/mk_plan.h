// Host-side schedule builder: per-CU instruction queues and the packed-weight
// stream layout.  Pure C++ (no HIP), so it also runs on machines without a GPU.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_internal.h"

namespace mk {

// Source matrices of the pack table: MatKind (mk_internal.h), layer * MATS_PER_LAYER + kind.

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
    uint32_t grow;       // global row index: mat_row_off[mat] + row (FP8: the row's scale)
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
    bool fp8 = false;
    // LM-head row-groups of two rows (2 rg, 2 rg + 1) with several batch rows (x read from LDS
    // per unit for every batch row): one x read then serves two rows
    bool lm_pairs = false;
    int epu = UNIT_ELEMS;                // weight elements per unit (1024 with FP8 codes)
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
    std::vector<uint32_t> mat_row_off;   // [n_mats + 1] global index of each matrix's row 0
    uint32_t rgs_off[4] = {0, 0, 0, 0};  // row-group scale table layout (Params::rgscale)
    uint32_t rgs_stride = 0;

    int lm_mat() const { return L * MATS_PER_LAYER; }
    // rows and columns of source matrix `mat`; false for an index past the LM head
    bool mat_shape(uint32_t mat, uint32_t& rows, uint32_t& cols) const {
        if (mat == (uint32_t)lm_mat()) {
            rows = V;
            cols = H;
            return true;
        }
        if (mat > (uint32_t)lm_mat()) return false;
        const uint32_t QD = Hq * D, KD = Hkv * D;
        switch (mat % MATS_PER_LAYER) {
        case MAT_WQ: rows = QD; cols = H; break;
        case MAT_WK: case MAT_WV: rows = KD; cols = H; break;
        case MAT_WO: rows = H; cols = QD; break;
        case MAT_GATE: case MAT_UP: rows = F; cols = H; break;
        default: rows = H; cols = F; break;  // MAT_DOWN
        }
        return true;
    }
    int n_mats() const { return L * MATS_PER_LAYER + 1; }
    // Up/gate rows of CU slot t: its share of every down-projection chunk, chunk after chunk
    // (one instruction per CU and layer; row-group i of it is row ug_row(t, i))
    uint32_t ug_share(int t, int c, uint32_t& r0) const {
        const int c0 = chunk_begin[c], len = chunk_begin[c + 1] - c0;
        r0 = (uint32_t)(c0 + (int)((long long)len * t / ncu));
        return (uint32_t)(c0 + (int)((long long)len * (t + 1) / ncu)) - r0;
    }
    uint32_t ug_count(int t) const {
        uint32_t n = 0, r0;
        for (int c = 0; c < n_chunk; ++c) n += ug_share(t, c, r0);
        return n;
    }
    uint32_t ug_row(int t, uint32_t i) const {
        uint32_t r0 = 0;
        for (int c = 0; c < n_chunk; ++c) {
            const uint32_t n = ug_share(t, c, r0);
            if (i < n) return r0 + i;
            i -= n;
        }
        return 0xffffffffu;  // past the CU's rows
    }
};

// FP8 row-group scale table (Params::rgscale) from per-row scales indexed by global row.
void build_rg_scales(const Plan& p, const std::vector<float>& row_scale, std::vector<float>& out);

// Checks the config against the kernels' limits; fills `err` on failure.
int validate_config(const mk_config& cfg, std::string& err);

// Builds the queues and stream layout for `ncu` workgroups.
int build_plan(const mk_config& cfg, int ncu, Plan& out, std::string& err);

// Checks that every output is produced exactly once per step, that every queue
// is in stage order (check_order), and simulates the queues (each instruction
// runs once everything it reads has been produced); returns false with a
// message on a coverage hole, a duplicate, an out-of-order queue or a deadlock.
bool check_plan(const Plan& p, std::string& err, bool check_order = true);

// Deliberate schedule defects for testing check_plan, planted in the first
// queue that has a place for them: 1 duplicates the queue's first instruction
// into the next CU's queue, 2 removes its first up/gate instruction, 3 swaps
// its last down-projection instruction with the later-stage instruction after
// it (the queue then waits on its own later work).  Returns false if no queue
// has a place for the defect.
bool mutate_plan(Plan& p, int mutation);

}  // namespace mk
