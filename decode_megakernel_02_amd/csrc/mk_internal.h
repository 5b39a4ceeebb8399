// Internal definitions shared by the host plan builder (mk_plan.cpp), the host
// API (mk_api.cpp) and the device code (mk_kernels.hip).  Not part of the ABI.
#pragma once
#include <stdint.h>

namespace mk {

// Workgroup shape: one workgroup per CU, NW compute waves and NLOAD helper
// waves: one weight loader (streams the packed weights of every compute wave
// into their LDS rings) and one gather wave (stages the cross-CU inputs of
// each instruction).
constexpr int NW = 8;                 // compute waves
constexpr int NLOAD = 2;              // helper waves: 1 weight loader + 1 gather wave
constexpr int WG_THREADS = 64 * (NW + NLOAD);
constexpr int UNIT_BYTES = 1024;      // one DMA: 64 lanes x 16 B
constexpr int UNIT_ELEMS = 512;       // bf16 per unit
constexpr int MAX_BATCH = 8;
constexpr int LDS_BYTES = 160 * 1024; // gfx950 LDS per CU
constexpr int SIDE_MAX_FLOATS = 2048; // cap of one LDS side buffer (epilogue inputs)
constexpr int MAX_SLOTS = 3;          // staged-input buffer sets
constexpr int GREEDY_BLOCKS = 32;     // workgroups per batch row of the greedy argmax

// Fused ops, in the order they appear inside one layer.  The page
// "Megakernels: Deleting the Kernel Boundary to Win Back Microseconds"
// (section "One launch, one interpreter") lists the same seven opcodes.
enum Op : uint16_t {
    OP_NONE = 0,
    OP_RMS_QKV_ROPE = 1,  // RMSNorm + fused QKV rows + RoPE + K/V append
    OP_ATTENTION = 2,     // split-KV partial attention for (row, KV group, split)
    OP_ATTN_REDUCE = 3,   // log-sum-exp merge of the splits of one (row, head)
    OP_O_PROJ_RES = 4,    // O projection + residual
    OP_RMS_UP_GATE = 5,   // RMSNorm + gate/up rows + SiLU product
    OP_DOWN_RES = 6,      // one K-chunk of down-proj for a CU's rows; the last chunk adds the residual
    OP_RMS_LM_HEAD = 7,   // final RMSNorm + LM head rows
};

constexpr int STAGES_PER_LAYER = 6;  // QKV, ATTN, REDUCE, O, UPGATE, DOWN; LM head last

// Weight matrices: layer matrices at layer * MATS_PER_LAYER + kind, the LM head last.
enum MatKind : uint32_t { MAT_WQ = 0, MAT_WK, MAT_WV, MAT_WO, MAT_GATE, MAT_UP, MAT_DOWN, MATS_PER_LAYER };
constexpr int FP8_UNIT_ELEMS = 1024;  // FP8 codes per unit

// GEMV rows of ku units take the batch-1 path (x slice in registers, a row's units read
// together) for these shapes, else the general path; the pack layout depends on it (the
// general path reads the two rows of a row-group alternately, unit by unit).
#if defined(__HIP__)
#define MK_INLINE __attribute__((host, device, always_inline)) inline  // inlined into the kernels' dispatch
#else
#define MK_INLINE inline
#endif
MK_INLINE constexpr bool batch1_path(int B, int ku, bool fp8) { return B == 1 && (ku == 2 || (ku == 4 && !fp8)); }

// One queue entry (16 bytes).  GEMV ops: row-groups [rg0, rg0 + nrg) of the
// op's row-group space, distributed round-robin over the NW compute waves
// (row-group i goes to wave i % NW); b = the instruction's unit-rows (the
// most weight units any one wave reads in it).  DOWN_RES: a = chunk.
// ATTENTION: a = batch row, b = KV group, rg0 = split.
// ATTN_REDUCE: a = batch row, b = query head.
struct Inst {
    uint16_t op;
    uint16_t layer;
    uint32_t rg0;
    uint32_t nrg;
    uint16_t a, b;
};
static_assert(sizeof(Inst) == 16, "Inst is 16 bytes");

// Everything the kernel reads, in one device-resident block.
struct Params {
    // model / run shape
    int32_t L, H, Hq, Hkv, D, F, V, B, max_seq;
    int32_t G;              // Hq / Hkv
    int32_t n_split, n_chunk;
    int32_t ku_h;           // units per row for K = H (padded to 512)
    int32_t ku_q;           // units per row for K = Hq*D
    int32_t ku_f;           // units per row for one down chunk (padded)
    int32_t xstride;        // floats per batch row in the LDS x buffer (max padded K)
    int32_t ring_units;     // ring slots (1 KB units) per compute wave
    int32_t xbuf_bytes;     // bytes of one of the two LDS x buffers
    int32_t side_floats;    // floats of each LDS side buffer (epilogue inputs staged by the gather
                            // wave); 0: epilogue inputs are read from global memory instead
    int32_t nslot;          // x / side buffer sets (1 to MAX_SLOTS; the host takes 1): the gather wave runs
                            // nslot - 1 instructions ahead
    int32_t res_stride;     // floats per batch row of the LDS residual rows (the CU's rows of the O and
                            // down projections, which are the same tile); 0: no resident rows
    int32_t ncu;            // workgroups in the grid
    float eps;
    float inv_sqrt_d;
    uint32_t spin_limit;    // bounded waits (watchdog)
    uint32_t ablate_op;     // ablation build: the opcode whose arithmetic is skipped (0: none)
    uint32_t lds_bytes;     // dynamic LDS of the step kernels (the NaN fill of the debug mode)
    int32_t chunk_begin[17];// down-proj chunk boundaries in [0, F], n_chunk + 1 entries

    // packed weights: per (cu, wave) stream of units
    const uint8_t* wstream;
    const uint64_t* stream_base;   // [ncu * NW] unit 0 of each stream; unit k at base + k * NW
    const Inst* insts;             // all queues back to back
    const uint32_t* queue_begin;   // [ncu + 1] index into insts
    const uint32_t* unit_off;      // [(queue_begin[cu] + pc + cu) * NW + w]: units before pc (pc in 0..len)
    const uint32_t* stage_pc;      // [ncu * (n_stages + 1)] first pc of each stage in each queue
    int32_t n_stages;

    // weights read in place
    const uint16_t* embed;         // [V][H] bf16 (token gather)
    const uint16_t* gain_attn;     // [L][H]
    const uint16_t* gain_mlp;      // [L][H]
    const uint16_t* gain_final;    // [H]
    const float* rope;             // [max_seq][D/2][2] (cos, sin)

    // tagged activations: 64-bit words {low: fp32 bits, high: step epoch}
    uint64_t* qkv;    // [L][B][Hkv][(G+2)*D]: the group's G query heads (after RoPE), then the
                      // new K row (after RoPE) and V row, both rounded to bf16 values
    uint64_t* part;   // [L][B][Hq][n_split][D+2]  (m, l, o[D])
    uint64_t* attn;   // [L][B][Hq*D]
    uint64_t* hmid;   // [L][B][H]   residual stream after the attention block
    uint64_t* act;    // [L][B][F]   SwiGLU output
    uint64_t* hout;   // [L][B][H]   residual stream after the MLP block (input of layer l+1)
    float* dacc;      // [B][H]      down-proj chunk accumulator, private to the row's owner wave
    const void* const* mats;  // unused by the step kernels (pack only)

    uint64_t* prof;   // [ncu][NW + NLOAD][8] cycle counters, or null
    uint64_t* trace;  // [total instructions][TRACE_SLOTS] timeline records, or null
    uint32_t* epoch;  // [ncu] per-workgroup step counter
    uint32_t* error;  // [8] device error record (code, wg, pc, op, wave, detail), abort flag at [7]

    // FP8 weights: the scales of the two rows of every row-group, {row 0, row 1} pairs (1 for a
    // row-group of one row), in row-group order: layer l's QKV pairs at l * rgs_stride +
    // rgs_off[0], its O rows at + rgs_off[1], gate/up rows at + rgs_off[2], down rows at +
    // rgs_off[3]; the LM head's rows at L * rgs_stride
    const float* rgscale;
    uint32_t rgs_off[4];
    uint32_t rgs_stride;
    int32_t fp8;          // weights packed as FP8 codes (units of 1024 elements)
    int32_t lm_pairs;     // LM-head row-groups are row pairs (2 rg, 2 rg + 1)

    // fused greedy decoding (mk_decode_step_greedy): arrival counter of the CUs (0 between
    // steps) and each CU's (max logit, lowest index) per batch row as two tagged words
    uint32_t* greedy_cnt;      // [1]
    uint64_t* greedy_pair;     // [ncu][MAX_BATCH][2]
};

// Kernel launch flags.
constexpr uint32_t KF_BUMP_EPOCH = 1u;  // last launch of a step: advance the per-workgroup epoch
constexpr uint32_t KF_INSTRUMENTED = 2u;  // run the kernel build that records profile counters / timelines
constexpr uint32_t KF_FP8 = 4u;           // run the kernel build for FP8 weights
constexpr uint32_t KF_GREEDY = 8u;        // single launch only: the build that also takes the argmax
constexpr uint32_t KF_ABLATE = 16u;       // single launch only: the build that can skip one opcode's math
constexpr uint32_t KF_POISON = 32u;       // debugging: fill the workgroup's LDS with NaN at launch
constexpr uint32_t KF_BATCHED = 64u;      // handle with several batch rows: the batched build of the step
constexpr int PROF_SLOTS = 8;          // counters per wave
// Timeline record per instruction (100 MHz real-time clock): [0] op | layer << 8 |
// a << 16 | b << 32 | cu << 48, then per compute wave w at [1 + 6w]: start,
// cross-CU inputs loaded, inputs ready, main loop done (before the epilogue
// or merge), end, ticks spent waiting for weight units; then the gather
// wave's start, all polled inputs current, inputs staged.
constexpr int TRACE_WAVE_SLOTS = 6;
constexpr int TRACE_SLOTS = 1 + TRACE_WAVE_SLOTS * NW + 3;


// Batched prefill (mk_prefill, mk_prefill_static): shapes, the caller's bf16
// weights (per-layer pointers read on the host at launch) and a workspace of
// fp32 rows for one chunk of positions (at most chunk positions of every
// batch row, M = B * chunk rows): X [M][H] residual, A [M][H] normalised
// input, QKV [M][Hq*D + 2*Hkv*D], O [M][Hq*D], G and U [M][F].  Prompt tokens
// outside [0, V) set *bad (when non-null) and the device error record err
// (when non-null; code 2, as a decode step does).
struct PrefillArgs {
    int L, H, Hq, Hkv, D, F, V, B, P, max_seq;
    int chunk;  // positions per pass through the layers
    float eps;
    const int32_t* tokens;  // [B][P]
    const uint16_t* embed;
    const uint16_t* final_norm;
    const uint16_t* lm_head;  // the embedding when tied
    const void* const* attn_norm;  // host arrays of L device pointers (mk_weights)
    const void* const* wq;
    const void* const* wk;
    const void* const* wv;
    const void* const* wo;
    const void* const* mlp_norm;
    const void* const* w_gate;
    const void* const* w_up;
    const void* const* w_down;
    const float* rope;  // [max_seq][D/2][2]
    uint16_t* kv;
    float* logits;  // [B][V]
    float *X, *A, *QKV, *O, *G, *U;
    uint32_t* bad;
    uint32_t* err;
};
// fp32 workspace floats of one prefill row (position of one batch row)
inline size_t prefill_row_floats(int H, int Hq, int Hkv, int D, int F) {
    return 2 * (size_t)H + 2 * (size_t)Hq * D + 2 * (size_t)Hkv * D + 2 * (size_t)F;
}
// Static prefill scratch of every device the library runs on (mk_prefill_static).
constexpr size_t PREFILL_SCRATCH_BYTES = (size_t)64 << 20;

}  // namespace mk
