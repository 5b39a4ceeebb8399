// Host side of the C ABI declared in include/mk.h: handle lifetime, device
// memory, weight packing, and the per-step launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_internal.h"
#include "mk_plan.h"

static_assert(MK_STEP_THREADS == mk::WG_THREADS, "public workgroup size matches the kernels");

namespace mk {
hipError_t launch_step(const Params* dev_params, int head_dim, int ncu, size_t lds_bytes, const int32_t* tokens,
                       const int32_t* positions, void* kv, float* logits, int stage, uint32_t flags,
                       hipStream_t stream);
hipError_t set_step_kernel_lds(size_t lds_bytes);
hipError_t launch_pack(const void* rows, uint32_t n, const uint16_t* const* mats, uint8_t* dst, int fp8,
                       const float* scales, hipStream_t stream);
hipError_t launch_poison(uint64_t* arena, size_t words, float* f0, size_t n0, float* f1, size_t n1,
                         hipStream_t stream);
hipError_t launch_row_amax(const uint16_t* w, uint32_t rows, uint32_t cols, uint16_t* out, hipStream_t stream);
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, int ncu, hipStream_t stream);
hipError_t launch_empty(int n_blocks, int n_threads, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);
hipError_t prefill_scratch_address(int device, void** out);
hipError_t launch_greedy(const float* logits, int B, int V, int32_t* tokens, int32_t* positions, uint64_t* part,
                         uint32_t* cnt, hipStream_t stream);
hipError_t launch_litmus(uint64_t* buf, int npairs, int rounds, int words, uint32_t spin_limit, uint32_t* result,
                         hipStream_t stream);
}  // namespace mk

using namespace mk;

struct mk_handle {
    mk_config cfg{};
    Plan plan;
    Params hp{};
    Params* dparams = nullptr;        // the single-launch step's parameter block
    Params* dparams_stage = nullptr;  // the per-op launches' block (its own LDS layout)
    size_t lds_bytes_stage = 0;
    std::vector<void*> allocs;  // everything hipMalloc'ed, freed in mk_destroy
    size_t lds_bytes = 0;
    bool loaded = false;
    std::string last_error;
    uint64_t* greedy_part = nullptr;  // [B][GREEDY_BLOCKS] per-slice (value, index) pairs
    uint32_t* greedy_cnt = nullptr;   // [B] finished slices of the current call (zero between calls)
    uint32_t ablate = 0;              // mk_set_ablation: opcode switched off in mk_decode_step (0: none)
    uint64_t* arena = nullptr;        // the tagged activation words (the debug NaN fill)
    size_t arena_words = 0;
    uint16_t* row_amax = nullptr;     // FP8: [rows of all matrices] largest |w| per row (bf16 bits)
    float* row_scale = nullptr;       // FP8: [rows of all matrices] scale of each row (pack input)
    void* prefill_ws = nullptr;       // mk_prefill's workspace, kept between calls
    size_t prefill_ws_bytes = 0;
    void* prefill_scratch = nullptr;  // device address of this device's static prefill scratch
};

static thread_local std::string g_create_error;
static constexpr uint32_t DEFAULT_SPIN_LIMIT = 1u << 25;  // polls before a wait gives up (seconds)
static constexpr size_t PREFILL_WS_MAX = (size_t)512 << 20;  // largest workspace mk_prefill keeps

namespace {

struct HipError {
    hipError_t e;
    const char* what;
};

#define HIPCHK(call)                                     \
    do {                                                 \
        hipError_t _e = (call);                          \
        if (_e != hipSuccess) throw HipError{_e, #call}; \
    } while (0)

template <class T>
T* dalloc(mk_handle* h, size_t count) {
    void* p = nullptr;
    if (count == 0) count = 1;
    hipError_t e = hipMalloc(&p, count * sizeof(T));
    if (e != hipSuccess) throw HipError{e, "hipMalloc"};
    h->allocs.push_back(p);
    return (T*)p;
}

template <class T>
T* dupload(mk_handle* h, const std::vector<T>& v) {
    T* d = dalloc<T>(h, v.size());
    if (!v.empty()) HIPCHK(hipMemcpy(d, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice));
    return d;
}

int fail(mk_handle* h, int code, const std::string& msg) {
    if (h) h->last_error = msg;
    else g_create_error = msg;
    return code;
}

int hip_fail(mk_handle* h, const HipError& e) {
    std::string msg = std::string(e.what) + ": " + hipGetErrorString(e.e);
    return fail(h, e.e == hipErrorOutOfMemory ? MK_ERR_OOM : MK_ERR_HIP, msg);
}

void free_all(mk_handle* h) {
    for (void* p : h->allocs) (void)hipFree(p);
    h->allocs.clear();
}

}  // namespace

extern "C" {

const char* mk_status_string(int s) {
    switch (s) {
    case MK_OK: return "ok";
    case MK_ERR_INVALID_ARG: return "invalid argument";
    case MK_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case MK_ERR_HIP: return "HIP runtime error";
    case MK_ERR_OOM: return "out of memory";
    case MK_ERR_STATE: return "invalid call order";
    case MK_ERR_DEVICE: return "device error record";
    default: return "unknown status";
    }
}

const char* mk_last_error(const mk_handle* h) { return h ? h->last_error.c_str() : g_create_error.c_str(); }

size_t mk_kv_cache_bytes(const mk_config* c) {
    if (!c) return 0;
    std::string err;
    if (validate_config(*c, err) != MK_OK) return 0;
    return (size_t)c->n_layers * 2 * c->batch * c->n_kv_heads * (size_t)c->max_seq * c->head_dim * 2;
}

int mk_schedule_inspect(const mk_config* cfg, int32_t n_cus, mk_schedule_info* out) {
    if (!cfg || !out || n_cus < 1) return fail(nullptr, MK_ERR_INVALID_ARG, "null argument or n_cus < 1");
    Plan p;
    std::string err;
    int rc;
    try {
        rc = build_plan(*cfg, n_cus, p, err);
    } catch (const std::bad_alloc&) {
        return fail(nullptr, MK_ERR_OOM, "host allocation failed");
    }
    if (rc != MK_OK) return fail(nullptr, rc, err);
    std::memset(out, 0, sizeof *out);
    out->n_cus = p.ncu;
    out->n_splits = p.n_split;
    out->n_chunks = p.n_chunk;
    out->total_insts = (int64_t)p.insts.size();
    for (int cu = 0; cu < p.ncu; ++cu)
        out->max_insts_per_cu = std::max(out->max_insts_per_cu, (int32_t)(p.queue_begin[cu + 1] - p.queue_begin[cu]));
    int64_t mx = 0, mn = INT64_MAX;
    for (uint64_t len : p.stream_len) {
        out->packed_weight_bytes += (int64_t)len * UNIT_BYTES;
        mx = std::max(mx, (int64_t)len * UNIT_BYTES);
        mn = std::min(mn, (int64_t)len * UNIT_BYTES);
    }
    out->max_stream_bytes_per_wave = mx;
    out->min_stream_bytes_per_wave = mn;
    out->launches_multikernel = p.n_stages;
    out->valid = check_plan(p, err) ? 1 : 0;
    if (!out->valid) g_create_error = err;
    return MK_OK;
}

int mk_schedule_selftest(const mk_config* cfg, int32_t n_cus, int32_t mutation) {
    if (!cfg || n_cus < 1 || mutation < 0 || mutation > 4)
        return fail(nullptr, MK_ERR_INVALID_ARG, "null config, n_cus < 1 or mutation outside 0..4");
    Plan p;
    std::string err;
    try {
        const int rc = build_plan(*cfg, n_cus, p, err);
        if (rc != MK_OK) return fail(nullptr, rc, err);
        if (mutation && !mutate_plan(p, mutation == 4 ? 3 : mutation))
            return fail(nullptr, MK_ERR_INVALID_ARG, "the schedule has no place for this defect");
        if (!check_plan(p, err, mutation != 4)) return fail(nullptr, MK_ERR_UNSUPPORTED_SHAPE, err);
    } catch (const std::bad_alloc&) {
        return fail(nullptr, MK_ERR_OOM, "host allocation failed");
    }
    g_create_error.clear();
    return MK_OK;
}

int mk_create(const mk_config* cfg, mk_handle** out) {
    if (!out) return fail(nullptr, MK_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!cfg) return fail(nullptr, MK_ERR_INVALID_ARG, "cfg is NULL");
    std::string err;
    int rc = validate_config(*cfg, err);
    if (rc != MK_OK) return fail(nullptr, rc, err);
    mk_handle* h = new (std::nothrow) mk_handle();
    if (!h) return fail(nullptr, MK_ERR_OOM, "host allocation failed");
    h->cfg = *cfg;
    try {
        int ndev = 0;
        HIPCHK(hipGetDeviceCount(&ndev));
        if (cfg->device < 0 || cfg->device >= ndev) {
            delete h;
            return fail(nullptr, MK_ERR_INVALID_ARG, "device ordinal out of range");
        }
        HIPCHK(hipSetDevice(cfg->device));
        // this device's static prefill scratch (mk_prefill_static), looked up with the device current
        HIPCHK(prefill_scratch_address(cfg->device, &h->prefill_scratch));
        int ncu_dev = 0;
        HIPCHK(hipDeviceGetAttribute(&ncu_dev, hipDeviceAttributeMultiprocessorCount, cfg->device));
        int ncu = cfg->n_cus ? cfg->n_cus : ncu_dev;
        if (ncu > ncu_dev) {
            delete h;
            return fail(nullptr, MK_ERR_INVALID_ARG, "n_cus exceeds the device's CU count");
        }
        Plan& p = h->plan;
        rc = build_plan(*cfg, ncu, p, err);
        if (rc == MK_OK && !check_plan(p, err)) rc = MK_ERR_UNSUPPORTED_SHAPE;
        if (rc != MK_OK) {
            delete h;
            return fail(nullptr, rc, err);
        }
        // LDS: rings, nslot x buffers (also scratch of attention/reduce), sync words, nslot side buffers
        const int xstride = std::max(std::max(p.ku_h, p.ku_q), p.ku_f) * p.epu;
        size_t xb = (size_t)p.B * xstride * 4;
        const size_t attn_scratch = (size_t)(p.G * p.D + 2 * p.D + NW * (p.D + 2) + NW * 64) * 4;
        const size_t red_scratch = (size_t)p.n_split * (p.D + 2) * 4;
        xb = std::max(xb, std::max(attn_scratch, red_scratch));
        xb = (xb + 15) / 16 * 16;
        const size_t sync_bytes = 512;
        // side buffers: RoPE cos/sin rows of the step's positions (QKV) or the
        // residual rows of a CU's O / down-projection rows
        const size_t max_rows = (size_t)((p.H + ncu - 1) / ncu);
        size_t side = std::max((size_t)p.B * p.D, (size_t)p.B * max_rows);
        if (side > SIDE_MAX_FLOATS) side = 0;  // too many rows per CU: epilogues read global memory
        const size_t side_bytes = (side * 4 + 15) / 16 * 16;
        // launch-resident rows: the step's RoPE rows [B][D], and (with side buffers) the CU's
        // residual rows [B][max_rows], which the single-launch step keeps in LDS across ops
        const int res_stride = side ? (int)max_rows : 0;
        const size_t keep_bytes = ((size_t)p.B * p.D * 4 + (size_t)p.B * res_stride * 4 + 15) / 16 * 16;
        // the batch-1 path reads a whole row of units at once; the general path one unit at a time
        const int ring_need = p.B == 1 ? std::max(2, std::max(std::max(p.ku_h, p.ku_q), p.ku_f)) : 2;
        auto rings_for = [&](int nslot) {
            const long budget = (long)LDS_BYTES - nslot * (long)(xb + side_bytes) - (long)sync_bytes - (long)keep_bytes;
            return (int)std::min<long>(32, budget / (NW * UNIT_BYTES));
        };
        // one buffer set: the gather wave stages an instruction's inputs once every compute wave is
        // done with the previous instruction, and the LDS of further sets goes to the weight rings.
        // Staging one or two instructions ahead (the kernel takes up to MAX_SLOTS sets) measured
        // slower on every workload.
        const int nslot = 1;
        const int ring_units = rings_for(nslot);
        if (ring_units < ring_need) {
            delete h;
            return fail(nullptr, MK_ERR_UNSUPPORTED_SHAPE, "batch x hidden too large for the LDS budget");
        }
        h->lds_bytes = (size_t)NW * ring_units * UNIT_BYTES + nslot * (xb + side_bytes) + sync_bytes + keep_bytes;
        // the per-op launches run one stage per launch, where staging ahead still pays: three buffer
        // sets when the rings keep at least 12 slots, else two when they keep 4 (and what the batch-1
        // path needs), else one
        int nslot_stage = rings_for(3) >= std::max(ring_need, 12) ? 3 : rings_for(2) >= std::max(ring_need, 4) ? 2 : 1;
        const int ring_units_stage = rings_for(nslot_stage);
        h->lds_bytes_stage =
            (size_t)NW * ring_units_stage * UNIT_BYTES + nslot_stage * (xb + side_bytes) + sync_bytes + keep_bytes;
        h->hp.lds_bytes = (uint32_t)h->lds_bytes;

        Params& hp = h->hp;
        hp.L = p.L; hp.H = p.H; hp.Hq = p.Hq; hp.Hkv = p.Hkv; hp.D = p.D; hp.F = p.F; hp.V = p.V; hp.B = p.B;
        hp.max_seq = p.max_seq; hp.G = p.G; hp.n_split = p.n_split; hp.n_chunk = p.n_chunk;
        hp.ku_h = p.ku_h; hp.ku_q = p.ku_q; hp.ku_f = p.ku_f; hp.xstride = xstride;
        hp.ring_units = ring_units; hp.xbuf_bytes = (int)xb; hp.ncu = ncu;
        hp.side_floats = (int)(side_bytes / 4);
        hp.nslot = nslot;
        hp.res_stride = res_stride;
        hp.eps = p.eps; hp.inv_sqrt_d = (float)(1.0 / std::sqrt((double)p.D));
        hp.spin_limit = DEFAULT_SPIN_LIMIT;

        for (int i = 0; i <= p.n_chunk; ++i) hp.chunk_begin[i] = p.chunk_begin[i];
        hp.n_stages = p.n_stages;
        hp.fp8 = p.fp8 ? 1 : 0;
        hp.lm_pairs = p.lm_pairs ? 1 : 0;
        if (p.fp8) {
            const size_t nrows = p.mat_row_off[(size_t)p.n_mats()];
            hp.rgscale = dalloc<float>(h, ((size_t)p.rgs_stride * p.L + p.V) * 2);
            for (int i = 0; i < 4; ++i) hp.rgs_off[i] = p.rgs_off[i];
            hp.rgs_stride = p.rgs_stride;
            h->row_amax = dalloc<uint16_t>(h, nrows);
            h->row_scale = dalloc<float>(h, nrows);
        }

        hp.wstream = dalloc<uint8_t>(h, (size_t)p.total_units * UNIT_BYTES);
        hp.stream_base = dupload(h, p.stream_base);
        hp.insts = dupload(h, p.insts);
        hp.queue_begin = dupload(h, p.queue_begin);
        hp.unit_off = dupload(h, p.unit_off);
        hp.stage_pc = dupload(h, p.stage_pc);
        hp.embed = dalloc<uint16_t>(h, (size_t)p.V * p.H);
        hp.gain_attn = dalloc<uint16_t>(h, (size_t)p.L * p.H);
        hp.gain_mlp = dalloc<uint16_t>(h, (size_t)p.L * p.H);
        hp.gain_final = dalloc<uint16_t>(h, (size_t)p.H);
        // RoPE table: angle p * theta^(-2i/D) in double, cos/sin rounded to fp32
        {
            const int half = p.D / 2;
            std::vector<float> rope((size_t)p.max_seq * half * 2);
            for (int i = 0; i < half; ++i) {
                const double f = std::pow((double)p.theta, -2.0 * i / p.D);
                for (int pos = 0; pos < p.max_seq; ++pos) {
                    const double a = (double)pos * f;
                    rope[((size_t)pos * half + i) * 2 + 0] = (float)std::cos(a);
                    rope[((size_t)pos * half + i) * 2 + 1] = (float)std::sin(a);
                }
            }
            hp.rope = dupload(h, rope);
        }
        // tagged activations (zeroed: tag 0 never matches a step epoch)
        const size_t B = p.B, L = p.L, H = p.H, QD = (size_t)p.Hq * p.D, KD = (size_t)p.Hkv * p.D;
        const size_t n_qkv = L * B * (QD + 2 * KD), n_part = L * B * p.Hq * p.n_split * (p.D + 2);
        const size_t n_attn = L * B * QD, n_h = L * B * H, n_act = L * B * p.F;
        const size_t words = n_qkv + n_part + n_attn + 2 * n_h + n_act;
        uint64_t* arena = dalloc<uint64_t>(h, words);
        HIPCHK(hipMemset(arena, 0, words * 8));
        h->arena = arena;
        h->arena_words = words;
        uint64_t* cur = arena;
        hp.qkv = cur; cur += n_qkv;
        hp.part = cur; cur += n_part;
        hp.attn = cur; cur += n_attn;
        hp.hmid = cur; cur += n_h;
        hp.act = cur; cur += n_act;
        hp.hout = cur; cur += n_h;
        hp.dacc = dalloc<float>(h, B * H);
        hp.mats = nullptr;
        hp.trace = nullptr;
        if (cfg->flags & MK_FLAG_TRACE) {
            const size_t n = p.insts.size() * TRACE_SLOTS;
            hp.trace = dalloc<uint64_t>(h, n);
            HIPCHK(hipMemset(hp.trace, 0, n * 8));
        }
        hp.prof = nullptr;
        if (cfg->flags & MK_FLAG_PROFILE) {
            const size_t n = (size_t)ncu * (NW + NLOAD) * PROF_SLOTS;
            hp.prof = dalloc<uint64_t>(h, n);
            HIPCHK(hipMemset(hp.prof, 0, n * 8));
        }
        hp.epoch = dalloc<uint32_t>(h, (size_t)ncu);
        HIPCHK(hipMemset(hp.epoch, 0, (size_t)ncu * 4));
        hp.error = dalloc<uint32_t>(h, 8);
        HIPCHK(hipMemset(hp.error, 0, 32));
        // fused greedy decoding: the CUs' arrival counter and their (max, index) pairs
        hp.greedy_cnt = dalloc<uint32_t>(h, 1);
        HIPCHK(hipMemset(hp.greedy_cnt, 0, 4));
        hp.greedy_pair = dalloc<uint64_t>(h, (size_t)ncu * MAX_BATCH * 2);
        HIPCHK(hipMemset(hp.greedy_pair, 0, (size_t)ncu * MAX_BATCH * 2 * 8));
        h->greedy_part = dalloc<uint64_t>(h, (size_t)B * GREEDY_BLOCKS);
        h->greedy_cnt = dalloc<uint32_t>(h, (size_t)B);
        HIPCHK(hipMemset(h->greedy_cnt, 0, (size_t)B * 4));
        h->dparams = dalloc<Params>(h, 1);
        HIPCHK(hipMemcpy(h->dparams, &hp, sizeof hp, hipMemcpyHostToDevice));
        Params hs = hp;
        hs.nslot = nslot_stage;
        hs.ring_units = ring_units_stage;
        hs.lds_bytes = (uint32_t)h->lds_bytes_stage;
        h->dparams_stage = dalloc<Params>(h, 1);
        HIPCHK(hipMemcpy(h->dparams_stage, &hs, sizeof hs, hipMemcpyHostToDevice));
        HIPCHK(set_step_kernel_lds(std::max(h->lds_bytes, h->lds_bytes_stage)));
        HIPCHK(hipDeviceSynchronize());
    } catch (const HipError& e) {
        int code = hip_fail(nullptr, e);
        free_all(h);
        delete h;
        return code;
    } catch (const std::bad_alloc&) {
        free_all(h);
        delete h;
        return fail(nullptr, MK_ERR_OOM, "host allocation failed");
    }
    *out = h;
    return MK_OK;
}

int mk_load_weights(mk_handle* h, const mk_weights* w, void* stream) {
    if (!h) return fail(nullptr, MK_ERR_INVALID_ARG, "handle is NULL");
    if (!w || !w->embed || !w->final_norm || !w->attn_norm || !w->wq || !w->wk || !w->wv || !w->wo ||
        !w->mlp_norm || !w->w_gate || !w->w_up || !w->w_down)
        return fail(h, MK_ERR_INVALID_ARG, "a weight pointer is NULL");
    const Plan& p = h->plan;
    if (!p.tied && !w->lm_head) return fail(h, MK_ERR_INVALID_ARG, "lm_head is NULL for an untied model");
    for (int l = 0; l < p.L; ++l)
        if (!w->attn_norm[l] || !w->wq[l] || !w->wk[l] || !w->wv[l] || !w->wo[l] || !w->mlp_norm[l] ||
            !w->w_gate[l] || !w->w_up[l] || !w->w_down[l])
            return fail(h, MK_ERR_INVALID_ARG, "a per-layer weight pointer is NULL");
    hipStream_t s = (hipStream_t)stream;
    void* d_rows = nullptr;
    void* d_mats = nullptr;
    try {
        HIPCHK(hipSetDevice(h->cfg.device));
        std::vector<const uint16_t*> mats((size_t)p.n_mats(), nullptr);
        for (int l = 0; l < p.L; ++l) {
            const size_t b = (size_t)l * MATS_PER_LAYER;
            mats[b + MAT_WQ] = (const uint16_t*)w->wq[l];
            mats[b + MAT_WK] = (const uint16_t*)w->wk[l];
            mats[b + MAT_WV] = (const uint16_t*)w->wv[l];
            mats[b + MAT_WO] = (const uint16_t*)w->wo[l];
            mats[b + MAT_GATE] = (const uint16_t*)w->w_gate[l];
            mats[b + MAT_UP] = (const uint16_t*)w->w_up[l];
            mats[b + MAT_DOWN] = (const uint16_t*)w->w_down[l];
        }
        mats[p.lm_mat()] = (const uint16_t*)(p.tied ? w->embed : w->lm_head);
        HIPCHK(hipMalloc(&d_rows, p.pack.size() * sizeof(PackRow)));
        HIPCHK(hipMalloc(&d_mats, mats.size() * sizeof(void*)));
        HIPCHK(hipMemcpyAsync(d_rows, p.pack.data(), p.pack.size() * sizeof(PackRow), hipMemcpyHostToDevice, s));
        HIPCHK(hipMemcpyAsync(d_mats, mats.data(), mats.size() * sizeof(void*), hipMemcpyHostToDevice, s));
        if (p.fp8) {
            // one scale per row, fp32(max|w_row| / 448) (1 for a zero row): the largest magnitude of
            // every row as bf16 bits on the device, the quotient on the host
            const size_t nrows = p.mat_row_off[(size_t)p.n_mats()];
            for (int m = 0; m < p.n_mats(); ++m) {
                uint32_t rows = 0, cols = 0;
                p.mat_shape((uint32_t)m, rows, cols);
                HIPCHK(launch_row_amax(mats[(size_t)m], rows, cols, h->row_amax + p.mat_row_off[(size_t)m], s));
            }
            std::vector<uint16_t> bits(nrows);
            HIPCHK(hipMemcpyAsync(bits.data(), h->row_amax, nrows * 2, hipMemcpyDeviceToHost, s));
            HIPCHK(hipStreamSynchronize(s));
            std::vector<float> scale(nrows);
            for (size_t r = 0; r < nrows; ++r) {
                const uint32_t f = (uint32_t)bits[r] << 16;
                float amax;
                std::memcpy(&amax, &f, 4);
                scale[r] = amax == 0.0f ? 1.0f : amax / 448.0f;
            }
            std::vector<float> rgs;
            build_rg_scales(p, scale, rgs);
            HIPCHK(hipMemcpyAsync(h->row_scale, scale.data(), nrows * 4, hipMemcpyHostToDevice, s));
            HIPCHK(hipMemcpyAsync((void*)h->hp.rgscale, rgs.data(), rgs.size() * 4, hipMemcpyHostToDevice, s));
            HIPCHK(hipStreamSynchronize(s));  // the host vectors go out of scope
        }
        HIPCHK(launch_pack(d_rows, (uint32_t)p.pack.size(), (const uint16_t* const*)d_mats, (uint8_t*)h->hp.wstream,
                           p.fp8 ? 1 : 0, h->row_scale, s));
        const size_t HB = (size_t)p.H * 2;
        HIPCHK(hipMemcpyAsync((void*)h->hp.embed, w->embed, (size_t)p.V * HB, hipMemcpyDeviceToDevice, s));
        for (int l = 0; l < p.L; ++l) {
            HIPCHK(hipMemcpyAsync((uint8_t*)h->hp.gain_attn + l * HB, w->attn_norm[l], HB, hipMemcpyDeviceToDevice, s));
            HIPCHK(hipMemcpyAsync((uint8_t*)h->hp.gain_mlp + l * HB, w->mlp_norm[l], HB, hipMemcpyDeviceToDevice, s));
        }
        HIPCHK(hipMemcpyAsync((void*)h->hp.gain_final, w->final_norm, HB, hipMemcpyDeviceToDevice, s));
        HIPCHK(hipStreamSynchronize(s));
        HIPCHK(hipFree(d_rows));
        d_rows = nullptr;
        HIPCHK(hipFree(d_mats));
        d_mats = nullptr;
    } catch (const HipError& e) {
        if (d_rows) (void)hipFree(d_rows);
        if (d_mats) (void)hipFree(d_mats);
        return hip_fail(h, e);
    }
    static_assert(sizeof(PackRow) == 40, "PackRow matches the device pack record");
    h->loaded = true;
    h->last_error.clear();
    return MK_OK;
}

static int step_args_ok(mk_handle* h, const int32_t* tokens, const int32_t* positions, void* kv, float* logits) {
    if (!h) return fail(nullptr, MK_ERR_INVALID_ARG, "handle is NULL");
    if (!tokens || !positions || !kv || !logits) return fail(h, MK_ERR_INVALID_ARG, "a step pointer is NULL");
    if (!h->loaded) return fail(h, MK_ERR_STATE, "mk_load_weights has not been called");
    return MK_OK;
}

// handles created with profiling or tracing run the instrumented kernel build, FP8 handles the FP8 one
static uint32_t instr_flag(const mk_handle* h) {
    return ((h->hp.prof || h->hp.trace) ? KF_INSTRUMENTED : 0u) | (h->hp.fp8 ? KF_FP8 : 0u) |
           ((h->cfg.flags & MK_FLAG_DEBUG_NAN) ? KF_POISON : 0u) | (h->hp.B > 1 ? KF_BATCHED : 0u);
}

// MK_FLAG_DEBUG_NAN: NaN into the step's scratch before its first launch
static hipError_t poison_before_step(mk_handle* h, float* logits, hipStream_t s) {
    if (!(h->cfg.flags & MK_FLAG_DEBUG_NAN)) return hipSuccess;
    return launch_poison(h->arena, h->arena_words, h->hp.dacc, (size_t)h->hp.B * h->hp.H, logits,
                         (size_t)h->hp.B * h->hp.V, s);
}

int mk_decode_step(mk_handle* h, const int32_t* tokens, const int32_t* positions, void* kv_cache, float* logits,
                   void* stream) {
    int rc = step_args_ok(h, tokens, positions, kv_cache, logits);
    if (rc != MK_OK) return rc;
    hipError_t e = poison_before_step(h, logits, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(h, HipError{e, "mk_poison_kernel launch"});
    e = launch_step(h->dparams, h->hp.D, h->hp.ncu, h->lds_bytes, tokens, positions, kv_cache, logits, -1,
                    KF_BUMP_EPOCH | instr_flag(h) | (h->ablate ? KF_ABLATE : 0u), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(h, HipError{e, "mk_step_kernel launch"});
    return MK_OK;
}

int mk_decode_step_greedy(mk_handle* h, int32_t* tokens, int32_t* positions, void* kv_cache, float* logits,
                          void* stream) {
    int rc = step_args_ok(h, tokens, positions, kv_cache, logits);
    if (rc != MK_OK) return rc;
    if (h->ablate) return fail(h, MK_ERR_STATE, "an ablation is set: use mk_decode_step");
    if (instr_flag(h) & KF_INSTRUMENTED)
        return fail(h, MK_ERR_STATE, "the fused greedy step has no profiling or tracing build");
    hipError_t e = poison_before_step(h, logits, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(h, HipError{e, "mk_poison_kernel launch"});
    e = launch_step(h->dparams, h->hp.D, h->hp.ncu, h->lds_bytes, tokens, positions, kv_cache, logits, -1,
                               KF_BUMP_EPOCH | KF_GREEDY | instr_flag(h), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(h, HipError{e, "mk_step_kernel launch (fused greedy)"});
    return MK_OK;
}

int mk_decode_step_multikernel(mk_handle* h, const int32_t* tokens, const int32_t* positions, void* kv_cache,
                               float* logits, void* stream) {
    int rc = step_args_ok(h, tokens, positions, kv_cache, logits);
    if (rc != MK_OK) return rc;
    const int ns = h->hp.n_stages;
    hipError_t e0 = poison_before_step(h, logits, (hipStream_t)stream);
    if (e0 != hipSuccess) return hip_fail(h, HipError{e0, "mk_poison_kernel launch"});
    for (int st = 0; st < ns; ++st) {
        hipError_t e = launch_step(h->dparams_stage, h->hp.D, h->hp.ncu, h->lds_bytes_stage, tokens, positions, kv_cache,
                                   logits, st, (st == ns - 1 ? KF_BUMP_EPOCH : 0u) | instr_flag(h), (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(h, HipError{e, "mk_step_kernel stage launch"});
    }
    return MK_OK;
}

int mk_set_ablation(mk_handle* h, int32_t opcode) {
    if (!h) return fail(nullptr, MK_ERR_INVALID_ARG, "handle is NULL");
    if (opcode < 0 || opcode > (int32_t)OP_RMS_LM_HEAD) return fail(h, MK_ERR_INVALID_ARG, "opcode outside 0..7");
    if (opcode && (instr_flag(h) & (KF_INSTRUMENTED | KF_FP8)))
        return fail(h, MK_ERR_STATE, "the ablation build has no FP8, profiling or tracing form");
    const uint32_t v = (uint32_t)opcode;
    try {
        HIPCHK(hipSetDevice(h->cfg.device));
        HIPCHK(hipDeviceSynchronize());  // no step may be reading the parameter block
        HIPCHK(hipMemcpy(&h->dparams->ablate_op, &v, sizeof v, hipMemcpyHostToDevice));
    } catch (const HipError& e) {
        return hip_fail(h, e);
    }
    h->ablate = v;
    h->hp.ablate_op = v;
    return MK_OK;
}

int mk_set_spin_limit(mk_handle* h, uint32_t spins) {
    if (!h) return fail(nullptr, MK_ERR_INVALID_ARG, "handle is NULL");
    h->hp.spin_limit = spins ? spins : DEFAULT_SPIN_LIMIT;
    try {
        HIPCHK(hipSetDevice(h->cfg.device));
        HIPCHK(hipDeviceSynchronize());  // no step may be reading the parameter block
        HIPCHK(hipMemcpy(&h->dparams->spin_limit, &h->hp.spin_limit, sizeof(uint32_t), hipMemcpyHostToDevice));
        HIPCHK(hipMemcpy(&h->dparams_stage->spin_limit, &h->hp.spin_limit, sizeof(uint32_t), hipMemcpyHostToDevice));
    } catch (const HipError& e) {
        return hip_fail(h, e);
    }
    return MK_OK;
}

int mk_debug_stage(mk_handle* h, int32_t stage, const int32_t* tokens, const int32_t* positions, void* kv_cache,
                   float* logits, void* stream) {
    int rc = step_args_ok(h, tokens, positions, kv_cache, logits);
    if (rc != MK_OK) return rc;
    if (stage < 0 || stage >= h->hp.n_stages) return fail(h, MK_ERR_INVALID_ARG, "stage outside [0, n_stages)");
    // the epoch advances, so nothing this launch writes is ever taken for a later step's data
    hipError_t e = launch_step(h->dparams_stage, h->hp.D, h->hp.ncu, h->lds_bytes_stage, tokens, positions, kv_cache,
                               logits, stage, KF_BUMP_EPOCH | instr_flag(h), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(h, HipError{e, "mk_step_kernel stage launch"});
    return MK_OK;
}

int mk_greedy_advance(mk_handle* h, const float* logits, int32_t* tokens, int32_t* positions, void* stream) {
    if (!h || !logits || !tokens || !positions) return fail(h, MK_ERR_INVALID_ARG, "null argument");
    hipError_t e = launch_greedy(logits, h->hp.B, h->hp.V, tokens, positions, h->greedy_part, h->greedy_cnt,
                                 (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(h, HipError{e, "mk_greedy_kernel launch"});
    return MK_OK;
}

int mk_read_probe(const void* buf, size_t bytes, void* sink, int n_cus, void* stream) {
    if (!buf || !sink || n_cus < 1 || n_cus > 4096 || bytes % 16 != 0 || ((uintptr_t)buf & 15) != 0)
        return fail(nullptr, MK_ERR_INVALID_ARG, "mk_read_probe: null buffer, n_cus outside 1..4096 or unaligned size/address");
    hipError_t e = launch_read_probe(buf, bytes, (uint32_t*)sink, n_cus, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(nullptr, HipError{e, "mk_read_probe_kernel launch"});
    return MK_OK;
}

int mk_litmus(int device, int32_t n_pairs, int32_t rounds, int32_t words, uint32_t spin_limit, uint32_t* result) {
    if (n_pairs < 1 || n_pairs > 512 || rounds < 1 || rounds > (1 << 20) || words < 1 || words > 1024 || !result)
        return fail(nullptr, MK_ERR_INVALID_ARG, "mk_litmus: n_pairs 1..512, rounds 1..2^20, words 1..1024, result non-NULL");
    const size_t nres = 3 + 3 * (size_t)n_pairs;
    uint64_t* buf = nullptr;
    uint32_t* dres = nullptr;
    hipStream_t s = nullptr;
    int rc = MK_OK;
    try {
        HIPCHK(hipSetDevice(device));
        HIPCHK(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
        HIPCHK(hipMalloc(&buf, (size_t)n_pairs * 2 * words * 8));
        HIPCHK(hipMalloc(&dres, nres * 4));
        HIPCHK(hipMemsetAsync(buf, 0, (size_t)n_pairs * 2 * words * 8, s));
        HIPCHK(hipMemsetAsync(dres, 0, nres * 4, s));
        HIPCHK(launch_litmus(buf, n_pairs, rounds, words, spin_limit, dres, s));
        HIPCHK(hipMemcpyAsync(result, dres, nres * 4, hipMemcpyDeviceToHost, s));
        HIPCHK(hipStreamSynchronize(s));
    } catch (const HipError& e) {
        rc = hip_fail(nullptr, e);
    }
    if (s) {
        (void)hipStreamSynchronize(s);
        (void)hipStreamDestroy(s);
    }
    if (buf) (void)hipFree(buf);
    if (dres) (void)hipFree(dres);
    return rc;
}

int mk_empty_launches(int n_launches, int n_blocks, int n_threads, void* stream) {
    if (n_launches < 1 || n_launches > 100000 || n_blocks < 1 || n_blocks > 65536 || n_threads < 1 || n_threads > 1024)
        return fail(nullptr, MK_ERR_INVALID_ARG, "mk_empty_launches: count, blocks or threads out of range");
    for (int i = 0; i < n_launches; ++i) {
        hipError_t e = launch_empty(n_blocks, n_threads, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(nullptr, HipError{e, "mk_empty_kernel launch"});
    }
    return MK_OK;
}

// ------------------------------------------------------------ graphs ------

struct mk_graph {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

static void graph_free(mk_graph* g) {
    if (!g) return;
    if (g->exec) (void)hipGraphExecDestroy(g->exec);
    if (g->graph) (void)hipGraphDestroy(g->graph);
    delete g;
}

int mk_graph_create(mk_handle* h, int32_t* tokens, int32_t* positions, void* kv_cache, float* logits, int n_steps,
                    uint32_t flags, mk_graph** out) {
    if (!out) return fail(h, MK_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    int rc = step_args_ok(h, tokens, positions, kv_cache, logits);
    if (rc != MK_OK) return rc;
    if (n_steps < 1 || n_steps > 4096) return fail(h, MK_ERR_INVALID_ARG, "n_steps outside 1..4096");
    if (flags & ~(MK_GRAPH_MULTIKERNEL | MK_GRAPH_EMPTY | MK_GRAPH_FUSED_GREEDY))
        return fail(h, MK_ERR_INVALID_ARG, "unknown graph flag");
    if ((flags & MK_GRAPH_FUSED_GREEDY) && ((flags & (MK_GRAPH_MULTIKERNEL | MK_GRAPH_EMPTY)) ||
                                            (instr_flag(h) & KF_INSTRUMENTED)))
        return fail(h, MK_ERR_INVALID_ARG, "MK_GRAPH_FUSED_GREEDY takes the plain single-launch step only");
    mk_graph* g = new (std::nothrow) mk_graph;
    if (!g) return fail(h, MK_ERR_OOM, "host allocation failed");
    hipStream_t cs = nullptr;
    try {
        // captured on a private stream (the legacy default stream cannot be captured)
        HIPCHK(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
        HIPCHK(hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal));
        const int ns = h->hp.n_stages;
        HipError first{hipSuccess, ""};
        for (int i = 0; i < n_steps && first.e == hipSuccess; ++i) {
            if (!(flags & MK_GRAPH_EMPTY)) {
                first = HipError{poison_before_step(h, logits, cs), "mk_poison_kernel launch"};
                if (first.e != hipSuccess) break;
            }
            if (flags & MK_GRAPH_EMPTY) {
                for (int st = 0; st < ns && first.e == hipSuccess; ++st)
                    first = HipError{launch_empty(h->hp.ncu, WG_THREADS, cs), "mk_empty_kernel launch"};
                continue;
            }
            if (flags & MK_GRAPH_MULTIKERNEL) {
                for (int st = 0; st < ns && first.e == hipSuccess; ++st)
                    first = HipError{launch_step(h->dparams_stage, h->hp.D, h->hp.ncu, h->lds_bytes_stage, tokens,
                                                 positions, kv_cache, logits, st,
                                                 (st == ns - 1 ? KF_BUMP_EPOCH : 0u) | instr_flag(h), cs),
                                     "mk_step_kernel stage launch"};
            } else if (flags & MK_GRAPH_FUSED_GREEDY) {
                first = HipError{launch_step(h->dparams, h->hp.D, h->hp.ncu, h->lds_bytes, tokens, positions, kv_cache,
                                             logits, -1, KF_BUMP_EPOCH | KF_GREEDY | instr_flag(h), cs),
                                 "mk_step_kernel launch (fused greedy)"};
                continue;  // the step itself advanced the tokens and positions
            } else {
                first = HipError{launch_step(h->dparams, h->hp.D, h->hp.ncu, h->lds_bytes, tokens, positions, kv_cache,
                                             logits, -1, KF_BUMP_EPOCH | instr_flag(h), cs),
                                 "mk_step_kernel launch"};
            }
            if (first.e == hipSuccess)
                first = HipError{launch_greedy(logits, h->hp.B, h->hp.V, tokens, positions, h->greedy_part,
                                               h->greedy_cnt, cs),
                                 "mk_greedy_kernel launch"};
        }
        hipGraph_t graph = nullptr;
        const hipError_t ec = hipStreamEndCapture(cs, &graph);  // ends the capture whatever happened above
        g->graph = graph;
        if (first.e != hipSuccess) throw first;
        if (ec != hipSuccess) throw HipError{ec, "hipStreamEndCapture"};
        HIPCHK(hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0));
        HIPCHK(hipStreamDestroy(cs));
        cs = nullptr;
    } catch (const HipError& e) {
        if (cs) (void)hipStreamDestroy(cs);
        graph_free(g);
        (void)hipGetLastError();
        return hip_fail(h, e);
    }
    *out = g;
    return MK_OK;
}

int mk_graph_launch(mk_graph* g, void* stream) {
    if (!g || !g->exec) return fail(nullptr, MK_ERR_INVALID_ARG, "graph is NULL");
    hipError_t e = hipGraphLaunch(g->exec, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(nullptr, HipError{e, "hipGraphLaunch"});
    return MK_OK;
}

int mk_graph_destroy(mk_graph* g) {
    graph_free(g);
    return MK_OK;
}

int mk_get_device_error(mk_handle* h, mk_device_error* out) {
    if (!h || !out) return fail(h, MK_ERR_INVALID_ARG, "null argument");
    uint32_t rec[8] = {0};
    try {
        HIPCHK(hipSetDevice(h->cfg.device));
        HIPCHK(hipDeviceSynchronize());
        HIPCHK(hipMemcpy(rec, h->hp.error, sizeof rec, hipMemcpyDeviceToHost));
        if (rec[0] || rec[7]) {
            HIPCHK(hipMemset(h->hp.error, 0, sizeof rec));
            // an aborted fused-greedy step may have left CUs counted in: start the count afresh
            HIPCHK(hipMemset(h->hp.greedy_cnt, 0, 4));
        }
    } catch (const HipError& e) {
        return hip_fail(h, e);
    }
    out->code = rec[0];
    out->workgroup = rec[1];
    out->pc = rec[2];
    out->opcode = rec[3];
    out->wave = rec[4];
    out->detail = rec[5];
    return rec[0] ? MK_ERR_DEVICE : MK_OK;
}

int mk_get_profile(mk_handle* h, uint64_t* counters, size_t n) {
    if (!h || !counters) return fail(h, MK_ERR_INVALID_ARG, "null argument");
    if (!h->hp.prof) return fail(h, MK_ERR_STATE, "handle was created without MK_FLAG_PROFILE");
    const size_t need = (size_t)h->hp.ncu * (NW + NLOAD) * PROF_SLOTS;
    if (n < need) return fail(h, MK_ERR_INVALID_ARG, "counter buffer too small");
    try {
        HIPCHK(hipSetDevice(h->cfg.device));
        HIPCHK(hipDeviceSynchronize());
        HIPCHK(hipMemcpy(counters, h->hp.prof, need * 8, hipMemcpyDeviceToHost));
    } catch (const HipError& e) {
        return hip_fail(h, e);
    }
    return MK_OK;
}

int mk_get_trace(mk_handle* h, uint64_t* records, size_t n) {
    if (!h || !records) return fail(h, MK_ERR_INVALID_ARG, "null argument");
    if (!h->hp.trace) return fail(h, MK_ERR_STATE, "handle was created without MK_FLAG_TRACE");
    const size_t need = h->plan.insts.size() * TRACE_SLOTS;
    if (n < need) return fail(h, MK_ERR_INVALID_ARG, "record buffer too small");
    try {
        HIPCHK(hipSetDevice(h->cfg.device));
        HIPCHK(hipDeviceSynchronize());
        HIPCHK(hipMemcpy(records, h->hp.trace, need * 8, hipMemcpyDeviceToHost));
    } catch (const HipError& e) {
        return hip_fail(h, e);
    }
    return MK_OK;
}

// Shared argument checks and launch arguments of mk_prefill / mk_prefill_static; chunk and the
// workspace pointers are filled in by the caller.
static int prefill_args(mk_handle* h, const mk_weights* w, const int32_t* tokens, int32_t n_tokens, void* kv_cache,
                        float* logits, PrefillArgs& a) {
    if (!h) return fail(nullptr, MK_ERR_INVALID_ARG, "handle is NULL");
    if (!w || !tokens || !kv_cache || !logits) return fail(h, MK_ERR_INVALID_ARG, "null argument");
    const Params& p = h->hp;
    if (h->cfg.flags & MK_FLAG_FP8_WEIGHTS)
        return fail(h, MK_ERR_UNSUPPORTED_SHAPE, "prefill runs on bf16 weights; the handle decodes FP8 weights");
    if (n_tokens < 1 || n_tokens > h->cfg.max_seq) return fail(h, MK_ERR_INVALID_ARG, "n_tokens must be in [1, max_seq]");
    const bool tied = h->cfg.tied_embeddings != 0;
    if (!w->embed || !w->final_norm || (!tied && !w->lm_head) || !w->attn_norm || !w->wq || !w->wk || !w->wv ||
        !w->wo || !w->mlp_norm || !w->w_gate || !w->w_up || !w->w_down)
        return fail(h, MK_ERR_INVALID_ARG, "a weight pointer is NULL");
    auto aligned = [](const void* q) { return q && ((uintptr_t)q & 15u) == 0; };
    bool ok = aligned(w->embed) && aligned(w->final_norm) && (tied || aligned(w->lm_head)) &&
              aligned(tokens) && aligned(kv_cache) && aligned(logits);
    for (int l = 0; l < p.L && ok; ++l)
        ok = aligned(w->attn_norm[l]) && aligned(w->wq[l]) && aligned(w->wk[l]) && aligned(w->wv[l]) &&
             aligned(w->wo[l]) && aligned(w->mlp_norm[l]) && aligned(w->w_gate[l]) && aligned(w->w_up[l]) &&
             aligned(w->w_down[l]);
    if (!ok) return fail(h, MK_ERR_INVALID_ARG, "every pointer must be non-NULL and 16-byte aligned");
    a = PrefillArgs{};
    a.L = p.L; a.H = p.H; a.Hq = p.Hq; a.Hkv = p.Hkv; a.D = p.D; a.F = p.F; a.V = p.V; a.B = p.B;
    a.P = n_tokens; a.max_seq = h->cfg.max_seq; a.eps = h->cfg.rms_eps;
    a.tokens = tokens;
    a.embed = (const uint16_t*)w->embed;
    a.final_norm = (const uint16_t*)w->final_norm;
    a.lm_head = (const uint16_t*)(tied ? w->embed : w->lm_head);
    a.attn_norm = w->attn_norm; a.wq = w->wq; a.wk = w->wk; a.wv = w->wv; a.wo = w->wo;
    a.mlp_norm = w->mlp_norm; a.w_gate = w->w_gate; a.w_up = w->w_up; a.w_down = w->w_down;
    a.rope = p.rope;
    a.kv = (uint16_t*)kv_cache;
    a.logits = logits;
    return MK_OK;
}

// Carves the chunk workspace (rows of prefill_row_floats) out of ws.
static void prefill_carve(PrefillArgs& a, void* ws) {
    const size_t M = (size_t)a.B * a.chunk, H = a.H, QD = (size_t)a.Hq * a.D, KD = (size_t)a.Hkv * a.D;
    float* f = (float*)ws;
    a.X = f; f += M * H;
    a.A = f; f += M * H;
    a.QKV = f; f += M * (QD + 2 * KD);
    a.O = f; f += M * QD;
    a.G = f; f += M * a.F;
    a.U = f; f += M * a.F;
    a.bad = (uint32_t*)f;
}

int mk_prefill(mk_handle* h, const mk_weights* w, const int32_t* tokens, int32_t n_tokens, void* kv_cache,
               float* logits, void* stream) {
    PrefillArgs a;
    int rc = prefill_args(h, w, tokens, n_tokens, kv_cache, logits, a);
    if (rc != MK_OK) return rc;
    const Params& p = h->hp;
    const size_t row = prefill_row_floats(p.H, p.Hq, p.Hkv, p.D, p.F) * 4;
    // as many positions per chunk as the kept workspace allows (all of them when it fits)
    const size_t per_pos = (size_t)p.B * row;
    size_t chunk = std::min<size_t>((size_t)n_tokens, std::max<size_t>(1, (PREFILL_WS_MAX - 256) / per_pos));
    const size_t need = chunk * per_pos + 256;
    hipStream_t s = (hipStream_t)stream;
    try {
        HIPCHK(hipSetDevice(h->cfg.device));
        if (h->prefill_ws_bytes < need) {  // grow the kept workspace (the only allocation)
            if (h->prefill_ws) {
                HIPCHK(hipStreamSynchronize(s));
                for (auto it = h->allocs.begin(); it != h->allocs.end(); ++it)
                    if (*it == h->prefill_ws) {
                        h->allocs.erase(it);
                        break;
                    }
                (void)hipFree(h->prefill_ws);
                h->prefill_ws = nullptr;
                h->prefill_ws_bytes = 0;
            }
            void* ws = nullptr;
            if (hipMalloc(&ws, need) != hipSuccess) {
                (void)hipGetLastError();
                return fail(h, MK_ERR_OOM, "prefill workspace allocation failed");
            }
            h->allocs.push_back(ws);
            h->prefill_ws = ws;
            h->prefill_ws_bytes = need;
        }
        a.chunk = (int)chunk;
        prefill_carve(a, h->prefill_ws);
        a.err = nullptr;
        HIPCHK(hipMemsetAsync(a.bad, 0, 4, s));
        HIPCHK(launch_prefill(a, s));
        uint32_t bad = 0;
        HIPCHK(hipMemcpyAsync(&bad, a.bad, 4, hipMemcpyDeviceToHost, s));
        HIPCHK(hipStreamSynchronize(s));
        if (bad) return fail(h, MK_ERR_INVALID_ARG, "a prompt token is outside [0, vocab)");
    } catch (const HipError& e) {
        return hip_fail(h, e);
    }
    return MK_OK;
}

int mk_prefill_static(mk_handle* h, const mk_weights* w, const int32_t* tokens, int32_t n_tokens, void* kv_cache,
                      float* logits, void* stream) {
    PrefillArgs a;
    int rc = prefill_args(h, w, tokens, n_tokens, kv_cache, logits, a);
    if (rc != MK_OK) return rc;
    const Params& p = h->hp;
    const size_t per_pos = (size_t)p.B * prefill_row_floats(p.H, p.Hq, p.Hkv, p.D, p.F) * 4;
    const size_t fit = PREFILL_SCRATCH_BYTES / per_pos;
    if (fit == 0)
        return fail(h, MK_ERR_UNSUPPORTED_SHAPE,
                    "one prompt position of every batch row needs more than the 64 MiB static prefill scratch");
    a.chunk = (int)std::min<size_t>((size_t)n_tokens, fit);
    prefill_carve(a, h->prefill_scratch);
    a.bad = nullptr;                     // no host readback: tokens out of range go to the error record
    a.err = (uint32_t*)h->hp.error;
    hipError_t e = hipSetDevice(h->cfg.device);
    if (e == hipSuccess) e = launch_prefill(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(h, HipError{e, "prefill launch"});
    return MK_OK;
}

int mk_destroy(mk_handle* h) {
    if (!h) return MK_OK;
    (void)hipSetDevice(h->cfg.device);
    (void)hipDeviceSynchronize();
    free_all(h);
    delete h;
    return MK_OK;
}

}  // extern "C"
