// Device code for gfx950 (MI355X): the persistent decode interpreter, its op
// bodies, and the weight-pack kernel.
//
// One workgroup per CU runs 8 compute waves and 8 loader waves.  Loader wave i
// streams compute wave i's packed weights (a contiguous byte stream laid out at
// load time in exactly the order wave i consumes them) from HBM into a private
// LDS ring with global->LDS DMA, ahead of the dependency waits: weights never
// depend on activations, so the next instructions' loads overlap the tail of
// the current one (the page "Megakernels: Deleting the Kernel Boundary to Win
// Back Microseconds", sections "One launch, one interpreter" and "Correctness
// without the free barrier": shared memory paging so that the next
// instruction's loads start early).
//
// Dependencies between CUs are carried by the data itself: every activation
// word that crosses CUs is a 64-bit {fp32 value, step epoch} pair written with
// one agent-coherent (sc1) store, and a consumer polls its inputs until every
// tag equals the current epoch.  The same section of that page rebuilds the
// kernel-boundary ordering with counters bumped after a fence; on MI355X an
// agent-scope release costs an L2 writeback per signal and a 256-way counter
// serialises its atomics, so tags replace both while keeping the guarantee
// that a consumer never reads data older than its producer's store.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_internal.h"

namespace mk {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

#define CBAR() asm volatile("" ::: "memory")

constexpr int MAXOUT = 8;  // DMA units in flight per loader wave

// ------------------------------------------------------------- primitives --

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// float -> bf16 bits, round to nearest even
__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <int ctrl, int row_mask>
__device__ __forceinline__ float dpp_mov(float v, float identity) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(v), ctrl, row_mask, 0xF, false));
}
// wave64 reductions with DPP (quad permutes, row mirrors, row broadcasts); the
// result is complete in lane 63 and broadcast with readlane.
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_mov<0xB1, 0xF>(x, 0.f);
    x += dpp_mov<0x4E, 0xF>(x, 0.f);
    x += dpp_mov<0x141, 0xF>(x, 0.f);
    x += dpp_mov<0x140, 0xF>(x, 0.f);
    x += dpp_mov<0x142, 0xA>(x, 0.f);
    x += dpp_mov<0x143, 0xC>(x, 0.f);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
__device__ __forceinline__ float wave_max(float x) {
    const float ninf = -__builtin_inff();
    x = fmaxf(x, dpp_mov<0xB1, 0xF>(x, ninf));
    x = fmaxf(x, dpp_mov<0x4E, 0xF>(x, ninf));
    x = fmaxf(x, dpp_mov<0x141, 0xF>(x, ninf));
    x = fmaxf(x, dpp_mov<0x140, 0xF>(x, ninf));
    x = fmaxf(x, dpp_mov<0x142, 0xA>(x, ninf));
    x = fmaxf(x, dpp_mov<0x143, 0xC>(x, ninf));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// tagged activation words: relaxed atomics at agent scope compile to sc1
// (agent-coherent) 8-byte stores and loads; an aligned 8-byte store is seen
// whole or not at all, so value and tag always travel together.
__device__ __forceinline__ void st_tag(uint64_t* p, float v, uint32_t tag) {
    __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tag(const uint64_t* p) {
    return __hip_atomic_load((uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t tag_of(uint64_t w) { return (uint32_t)(w >> 32); }
__device__ __forceinline__ float val_of(uint64_t w) { return __uint_as_float((uint32_t)w); }

// LDS sync words between waves of one workgroup.  LDS requests of one wave
// complete in order, so a data write followed by a flag write is observed in
// that order by any wave that reads the flag and then the data.
__device__ __forceinline__ uint32_t lds_ld(const uint32_t* p) {
    return __hip_atomic_load((uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// The loader wave issues LDS DMA; the compiler would guard its own LDS
// accesses with vmcnt(0) waits (the DMA may alias them), so the loader touches
// its sync words through inline asm instead.
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const lds_void*)p; }
__device__ __forceinline__ uint32_t asm_lds_ld(uint32_t a) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
    return v;
}
__device__ __forceinline__ void asm_lds_st(uint32_t a, uint32_t v) {
    asm volatile("ds_write_b32 %0, %1" ::"v"(a), "v"(v) : "memory");
}
// wait until at most n vector-memory operations of this wave are outstanding
__device__ __forceinline__ void wait_vm_le(uint32_t n) {
    switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    }
}
static_assert(MAXOUT == 8, "wait_vm_le covers 0..7");

// ------------------------------------------------------------ wave context --

struct Ctx {
    const Params* p;
    int cu, wave, lane;
    uint32_t epoch;
    uint32_t pc;       // instruction index in this CU's queue (for error records)
    uint32_t op;
    bool aborted;
};

__device__ __forceinline__ bool abort_flag(const Params* p) {
    return __hip_atomic_load(&p->error[7], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}
__device__ __forceinline__ void record_error_rec(uint32_t* e, uint32_t code, uint32_t cu, uint32_t pc, uint32_t op,
                                             uint32_t wave, uint32_t detail) {
    if (atomicCAS(&e[0], 0u, code) == 0u) {
        e[1] = cu;
        e[2] = pc;
        e[3] = op;
        e[4] = wave;
        e[5] = detail;
    }
    __hip_atomic_store(&e[7], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void record_error(Ctx& cx, uint32_t code, uint32_t detail) {
    record_error_rec(cx.p->error, code, (uint32_t)cx.cu, cx.pc, cx.op, (uint32_t)cx.wave, detail);
    cx.aborted = true;
}
// one iteration of a bounded wait; returns false once the wait must give up
__device__ __forceinline__ bool keep_waiting(Ctx& cx, uint32_t& spins, uint32_t detail) {
    if (cx.aborted) return false;
    ++spins;
    if ((spins & 63u) == 0u && abort_flag(cx.p)) {
        cx.aborted = true;
        return false;
    }
    if (spins > cx.p->spin_limit) {
        record_error(cx, 1u, detail);
        return false;
    }
    __builtin_amdgcn_s_sleep(1);
    return true;
}

// ---------------------------------------------------------------- LDS map --

struct Lds {
    uint8_t* ring;      // [NW][ring_units][1024]
    float* xbuf[2];     // two x buffers of xbuf_bytes each
    uint32_t* landed;   // [NW] units landed in each compute wave's ring
    uint32_t* consumed; // [NW] units consumed
    uint32_t* bar;      // compute-wave barrier counter
    float* red;         // [MAX_BATCH][NW] partial sums of squares
};
__device__ __forceinline__ Lds lds_map(uint8_t* smem, const Params& p) {
    Lds m;
    m.ring = smem;
    size_t off = (size_t)NW * p.ring_units * UNIT_BYTES;
    m.xbuf[0] = (float*)(smem + off);
    m.xbuf[1] = (float*)(smem + off + p.xbuf_bytes);
    uint32_t* sync = (uint32_t*)(smem + off + 2 * (size_t)p.xbuf_bytes);
    m.landed = sync;
    m.consumed = sync + NW;
    m.bar = sync + 2 * NW;
    m.red = (float*)(sync + 2 * NW + 4);
    return m;
}

// barrier among the NW compute waves (loader waves never join it)
__device__ __forceinline__ void cbar(Ctx& cx, const Lds& s, uint32_t& seq) {
    seq += NW;
    CBAR();
    if (cx.lane == 0) __hip_atomic_fetch_add(s.bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    uint32_t spins = 0;
    while (lds_ld(s.bar) < seq)
        if (!keep_waiting(cx, spins, 0xBA000000u | seq)) break;
    CBAR();
}

// ------------------------------------------------------------- loader wave --

// Streams units [ub, ue) of compute wave w's stream into its ring.  Never
// blocks while DMA is in flight: when the ring is full it retires the oldest
// outstanding unit instead, so it cannot wait on the compute wave in a cycle.
__device__ __forceinline__ void loader(Ctx& cx, const Lds& s, int w, uint32_t ub, uint32_t ue) {
    const Params& p = *cx.p;
    const uint32_t n = ue - ub, ru = (uint32_t)p.ring_units;
    const uint8_t* src = p.wstream + (p.stream_base[cx.cu * NW + w] + ub) * (uint64_t)UNIT_BYTES + cx.lane * 16;
    uint8_t* ring = s.ring + (size_t)w * ru * UNIT_BYTES;
    const uint32_t a_landed = lds_addr(&s.landed[w]), a_consumed = lds_addr(&s.consumed[w]);
    uint32_t issued = 0, done = 0, slot = 0, spins = 0;
    while (done < n) {
        const uint32_t cons = asm_lds_ld(a_consumed);
        while (issued < n && issued - done < (uint32_t)MAXOUT && issued < cons + ru) {
            __builtin_amdgcn_global_load_lds((const glb_void*)(src + (uint64_t)issued * UNIT_BYTES),
                                             (lds_void*)(ring + (size_t)slot * UNIT_BYTES), 16, 0, 0);
            ++issued;
            slot = slot + 1 == ru ? 0 : slot + 1;
        }
        if (issued > done) {
            wait_vm_le(issued - done - 1);  // the oldest outstanding unit has landed
            ++done;
            asm_lds_st(a_landed, done);
            spins = 0;
        } else if (!keep_waiting(cx, spins, 0x10000000u | done)) {
            break;
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ------------------------------------------------------------ compute side --

struct Stream {  // compute wave's read cursor in its ring
    uint32_t unit;  // units consumed in this launch
    uint32_t slot;
};

__device__ __forceinline__ uint4 ring_take(Ctx& cx, const Lds& s, Stream& st) {
    uint32_t spins = 0;
    while (lds_ld(&s.landed[cx.wave]) <= st.unit)
        if (!keep_waiting(cx, spins, 0x20000000u | st.unit)) break;
    CBAR();
    const uint4 v = *(const uint4*)(s.ring + ((size_t)cx.wave * cx.p->ring_units + st.slot) * UNIT_BYTES + cx.lane * 16);
    return v;
}
__device__ __forceinline__ void ring_release(Ctx& cx, const Lds& s, Stream& st) {
    ++st.unit;
    st.slot = st.slot + 1 == (uint32_t)cx.p->ring_units ? 0 : st.slot + 1;
    CBAR();
    lds_st(&s.consumed[cx.wave], st.unit);
}

// x buffer layout per batch row: [half][chunk][4] with element k in half
// (k % 8) / 4, chunk k / 8, position k % 4, so a lane's 8 elements of one unit
// are two 16-byte reads at consecutive addresses across lanes.
__device__ __forceinline__ int xidx(const Params& p, int b, int k) {
    return b * p.xstride + ((k & 4) ? (p.xstride >> 1) : 0) + (k >> 3) * 4 + (k & 3);
}

__device__ __forceinline__ float dot8(const uint4 w, const float4 a, const float4 b) {
    float s = bf_lo(w.x) * a.x;
    s = fmaf(bf_hi(w.x), a.y, s);
    s = fmaf(bf_lo(w.y), a.z, s);
    s = fmaf(bf_hi(w.y), a.w, s);
    s = fmaf(bf_lo(w.z), b.x, s);
    s = fmaf(bf_hi(w.z), b.y, s);
    s = fmaf(bf_lo(w.w), b.z, s);
    s = fmaf(bf_hi(w.w), b.w, s);
    return s;
}

// Reads n tagged words *addr(i) (thread t of the 512 compute threads takes
// i = t, t+512, ...), waiting until each carries this step's epoch, and hands
// (i, value) to put.  Loads are issued eight at a time so latencies overlap.
template <class Addr, class Put>
__device__ __forceinline__ void acquire(Ctx& cx, int n, Addr&& addr, Put&& put) {
    const int t = cx.wave * 64 + cx.lane;
    constexpr int NT = NW * 64;
    for (int i0 = t; i0 < n; i0 += 8 * NT) {
        uint64_t w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = i0 + j * NT;
            w[j] = i < n ? ld_tag(addr(i)) : ((uint64_t)cx.epoch << 32);
        }
        uint32_t spins = 0;
        while (true) {
            bool ok = true;
#pragma unroll
            for (int j = 0; j < 8; ++j) ok &= tag_of(w[j]) == cx.epoch;
            if (ok) break;
            if (!keep_waiting(cx, spins, 0x30000000u | (uint32_t)i0)) break;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (tag_of(w[j]) != cx.epoch) w[j] = ld_tag(addr(i0 + j * NT));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = i0 + j * NT;
            if (i < n) put(i, val_of(w[j]));
        }
    }
}

// Poll a single tagged word (epilogue inputs that were produced long before).
__device__ __forceinline__ float wait_word(Ctx& cx, const uint64_t* p) {
    uint64_t w = ld_tag(p);
    uint32_t spins = 0;
    while (tag_of(w) != cx.epoch) {
        if (!keep_waiting(cx, spins, 0x40000000u)) break;
        w = ld_tag(p);
    }
    return val_of(w);
}

struct RowOut {
    float mine[2];  // row r's dot product for batch row `lane` (lanes < B)
};

// Dot products of one row-group (NROWS = 1 or 2 rows of ku units each) with x
// for every batch row; weights come from the ring.
template <int NROWS>
__device__ __forceinline__ void rowgroup_dot(Ctx& cx, const Lds& s, Stream& st, const float* xb, int ku, RowOut& out) {
    const Params& p = *cx.p;
    const int B = p.B;
#pragma unroll
    for (int r = 0; r < NROWS; ++r) {
        float acc[MAX_BATCH];
#pragma unroll
        for (int b = 0; b < MAX_BATCH; ++b) acc[b] = 0.f;
        for (int u = 0; u < ku; ++u) {
            const uint4 w = ring_take(cx, s, st);
            const int c = u * 64 + cx.lane;  // 8-element chunk index
#pragma unroll
            for (int b = 0; b < MAX_BATCH; ++b) {
                if (b < B) {
                    const float4* xr = (const float4*)(xb + b * p.xstride);
                    const float4 lo = xr[c], hi = xr[(p.xstride >> 3) + c];
                    acc[b] += dot8(w, lo, hi);
                }
            }
            ring_release(cx, s, st);
        }
        float mine = 0.f;
#pragma unroll
        for (int b = 0; b < MAX_BATCH; ++b) {
            if (b < B) {
                const float t = wave_sum(acc[b]);
                mine = cx.lane == b ? t : mine;
            }
        }
        out.mine[r] = mine;
    }
}

// Zero x[b][k] for k in [kvalid, kpad) (padding multiplies zero weights; NaN-free).
__device__ __forceinline__ void x_pad(Ctx& cx, float* xb, int kvalid, int kpad) {
    const Params& p = *cx.p;
    const int t = cx.wave * 64 + cx.lane;
    for (int b = 0; b < p.B; ++b)
        for (int k = kvalid + t; k < kpad; k += NW * 64) xb[xidx(p, b, k)] = 0.f;
}

// Finish an RMSNorm input held raw in LDS: after a barrier, each thread sums
// the squares of its elements of every batch row and multiplies them by the
// gain in place; per-wave partials go through LDS (fixed summation order) and
// lane b returns 1/sqrt(mean(h_b^2) + eps).  Two compute-wave barriers.
__device__ __forceinline__ float rms_finish(Ctx& cx, const Lds& s, uint32_t& seq, float* xb, const uint16_t* gain,
                                            int K) {
    const Params& p = *cx.p;
    const int t = cx.wave * 64 + cx.lane;
    cbar(cx, s, seq);
    for (int b = 0; b < p.B; ++b) {
        float ss = 0.f;
        for (int k = t; k < K; k += NW * 64) {
            float* x = xb + xidx(p, b, k);
            const float v = *x;
            ss = fmaf(v, v, ss);
            *x = v * bf2f(gain[k]);
        }
        ss = wave_sum(ss);
        if (cx.lane == 0) s.red[b * NW + cx.wave] = ss;
    }
    cbar(cx, s, seq);
    float my = 0.f;
    if (cx.lane < p.B) {
        float tot = 0.f;
        for (int w = 0; w < NW; ++w) tot += s.red[cx.lane * NW + w];
        my = 1.0f / sqrtf(tot / (float)K + p.eps);
    }
    return my;
}

struct Step {  // per-launch batch inputs, lane b holds row b
    int tok, pos;
    const int32_t* tokens;
    const int32_t* positions;
    uint16_t* kv;
    float* logits;
};

// ------------------------------------------------------------ GEMV ops ------

__device__ __forceinline__ void op_gemv(Ctx& cx, const Lds& s, Stream& st, uint32_t& seq, const Inst& in, float* xb,
                                        const Step& sp) {
    const Params& p = *cx.p;
    const int B = p.B, H = p.H, l = in.layer;
    int ku, kvalid;
    // ---- input vector (raw values) into LDS
    switch (in.op) {
    case OP_RMS_QKV_ROPE:
    case OP_RMS_LM_HEAD: {
        ku = p.ku_h;
        kvalid = H;
        const int src_layer = in.op == OP_RMS_LM_HEAD ? p.L : l;  // residual stream entering this layer
        if (src_layer == 0) {
            const int t = cx.wave * 64 + cx.lane;
            for (int b = 0; b < B; ++b) {
                const int tok = sp.tokens[b];
                for (int k = t; k < H; k += NW * 64) xb[xidx(p, b, k)] = bf2f(p.embed[(size_t)tok * H + k]);
            }
        } else {
            const uint64_t* src = p.hout + (size_t)(src_layer - 1) * B * H;
            acquire(cx, B * H, [&](int i) { return src + i; }, [&](int i, float v) {
                const int b = i / H;
                xb[xidx(p, b, i - b * H)] = v;
            });
        }
        break;
    }
    case OP_RMS_UP_GATE: {
        ku = p.ku_h;
        kvalid = H;
        const uint64_t* src = p.hmid + (size_t)l * B * H;
        acquire(cx, B * H, [&](int i) { return src + i; }, [&](int i, float v) {
            const int b = i / H;
            xb[xidx(p, b, i - b * H)] = v;
        });
        break;
    }
    case OP_O_PROJ_RES: {
        ku = p.ku_q;
        const int K = p.Hq * p.D;
        kvalid = K;
        const uint64_t* src = p.attn + (size_t)l * B * K;
        acquire(cx, B * K, [&](int i) { return src + i; }, [&](int i, float v) {
            const int b = i / K;
            xb[xidx(p, b, i - b * K)] = v;
        });
        break;
    }
    default: {  // OP_DOWN_RES: chunk a of the SwiGLU output
        ku = p.ku_f;
        const int c0 = p.chunk_begin[in.a], K = p.chunk_begin[in.a + 1] - c0;
        kvalid = K;
        const uint64_t* src = p.act + (size_t)l * B * p.F + c0;
        acquire(cx, B * K, [&](int i) { const int b = i / K; return src + (size_t)b * p.F + (i - b * K); },
                [&](int i, float v) {
                    const int b = i / K;
                    xb[xidx(p, b, i - b * K)] = v;
                });
        break;
    }
    }
    x_pad(cx, xb, kvalid, ku * UNIT_ELEMS);
    float scale = 1.f;  // lane b: RMSNorm scale of batch row b
    if (in.op == OP_RMS_QKV_ROPE || in.op == OP_RMS_LM_HEAD) {
        scale = rms_finish(cx, s, seq, xb, in.op == OP_RMS_LM_HEAD ? p.gain_final : p.gain_attn + (size_t)l * H, H);
    } else if (in.op == OP_RMS_UP_GATE) {
        scale = rms_finish(cx, s, seq, xb, p.gain_mlp + (size_t)l * H, H);
    } else {
        cbar(cx, s, seq);
    }
    if (cx.aborted) return;

    // ---- this wave's row-groups; lane b < B finishes batch row b
    const int D = p.D, half = D / 2;
    const bool lane_row = cx.lane < B;
    const int b = lane_row ? cx.lane : 0;
    for (uint32_t i = cx.wave; i < in.nrg; i += NW) {
        const uint32_t rg = in.rg0 + i;
        RowOut o;
        switch (in.op) {
        case OP_RMS_QKV_ROPE: {
            rowgroup_dot<2>(cx, s, st, xb, ku, o);
            if (lane_row) {
                const int pos = sp.pos;
                const float y1 = o.mine[0] * scale, y2 = o.mine[1] * scale;
                const int G = p.G, PG = (G + 2) * half;
                const int g = rg / PG, t = rg % PG;
                if (t < (G + 1) * half) {  // q or k: rotate the pair (ii, ii + D/2)
                    const int ii = t < G * half ? t % half : t - G * half;
                    const float2 cs = *(const float2*)(p.rope + ((size_t)pos * half + ii) * 2);
                    const float r1 = y1 * cs.x - y2 * cs.y, r2 = y2 * cs.x + y1 * cs.y;
                    if (t < G * half) {
                        const int head = g * G + t / half;
                        uint64_t* q = p.q + ((size_t)l * B + b) * p.Hq * D + head * D;
                        st_tag(q + ii, r1, cx.epoch);
                        st_tag(q + ii + half, r2, cx.epoch);
                    } else {
                        const uint16_t k1 = f2bf(r1), k2 = f2bf(r2);
                        uint16_t* kc = sp.kv + ((((size_t)l * 2 + 0) * B + b) * p.Hkv + g) * (size_t)p.max_seq * D + (size_t)pos * D;
                        kc[ii] = k1;
                        kc[ii + half] = k2;
                        uint64_t* kn = p.knew + ((size_t)l * B + b) * p.Hkv * D + g * D;
                        st_tag(kn + ii, bf2f(k1), cx.epoch);
                        st_tag(kn + ii + half, bf2f(k2), cx.epoch);
                    }
                } else {  // v: no rotation
                    const int ii = t - (G + 1) * half;
                    const uint16_t v1 = f2bf(y1), v2 = f2bf(y2);
                    uint16_t* vc = sp.kv + ((((size_t)l * 2 + 1) * B + b) * p.Hkv + g) * (size_t)p.max_seq * D + (size_t)pos * D;
                    vc[ii] = v1;
                    vc[ii + half] = v2;
                    uint64_t* vn = p.vnew + ((size_t)l * B + b) * p.Hkv * D + g * D;
                    st_tag(vn + ii, bf2f(v1), cx.epoch);
                    st_tag(vn + ii + half, bf2f(v2), cx.epoch);
                }
            }
            break;
        }
        case OP_O_PROJ_RES: {
            // residual stream entering layer l (complete before this layer's QKV began)
            float hin = 0.f;
            if (lane_row) {
                if (l == 0) hin = bf2f(p.embed[(size_t)sp.tok * H + rg]);
                else hin = wait_word(cx, p.hout + ((size_t)(l - 1) * B + b) * H + rg);
            }
            rowgroup_dot<1>(cx, s, st, xb, ku, o);
            if (lane_row) st_tag(p.hmid + ((size_t)l * B + b) * H + rg, hin + o.mine[0], cx.epoch);
            break;
        }
        case OP_RMS_UP_GATE: {
            rowgroup_dot<2>(cx, s, st, xb, ku, o);
            if (lane_row) {
                const float gt = o.mine[0] * scale, up = o.mine[1] * scale;
                const float a = gt / (1.0f + __expf(-gt)) * up;  // silu(gate) * up
                st_tag(p.act + ((size_t)l * B + b) * p.F + rg, a, cx.epoch);
            }
            break;
        }
        case OP_DOWN_RES: {
            const bool first = in.a == 0, last = in.a == p.n_chunk - 1;
            float hm = 0.f;
            if (last && lane_row) hm = wait_word(cx, p.hmid + ((size_t)l * B + b) * H + rg);
            rowgroup_dot<1>(cx, s, st, xb, ku, o);
            if (lane_row) {
                float* acc = p.dacc + (size_t)b * H + rg;  // written and read only by this wave's lane b
                const float v = o.mine[0] + (first ? 0.f : *acc);
                if (last) st_tag(p.hout + ((size_t)l * B + b) * H + rg, hm + v, cx.epoch);
                else *acc = v;
            }
            break;
        }
        default: {  // OP_RMS_LM_HEAD
            rowgroup_dot<1>(cx, s, st, xb, ku, o);
            if (lane_row) sp.logits[(size_t)b * p.V + rg] = o.mine[0] * scale;
            break;
        }
        }
        if (cx.aborted) return;
    }
}

// ------------------------------------------------------- attention ops ------

// Split-KV partial attention of query heads g*G .. g*G+G-1 of batch row b over
// keys [j0, j1) of split s: writes (m, l, o[D]) with m the max score, l the
// sum of exp(score - m) and o the exp-weighted sum of V rows (unnormalised).
__device__ __forceinline__ void op_attention(Ctx& cx, const Lds& s, uint32_t& seq, const Inst& in, float* xb, const Step& sp) {
    const Params& p = *cx.p;
    const int B = p.B, D = p.D, G = p.G, l = in.layer, b = in.a, g = in.b, split = (int)in.rg0;
    const int pos = sp.positions[b];
    const int S = pos + 1;
    const int j0 = (int)((long long)split * S / p.n_split), j1 = (int)((long long)(split + 1) * S / p.n_split);
    // LDS scratch inside this instruction's x buffer
    float* qs = xb;                  // [G][D], pre-scaled by 1/sqrt(D)
    float* kn = qs + G * D;          // [D] new K row (bf16 values)
    float* vn = kn + D;              // [D] new V row
    float* stt = vn + D;             // [NW][D + 2] per-wave (m, l, o)
    float* ev = stt + NW * (D + 2);  // [NW][64] exp weights of the current key block
    // q of the group's heads, then the new K and V rows, in one polled read
    const uint64_t* qsrc = p.q + ((size_t)l * B + b) * p.Hq * D + (size_t)g * G * D;
    const uint64_t* ksrc = p.knew + ((size_t)l * B + b) * p.Hkv * D + (size_t)g * D;
    const uint64_t* vsrc = p.vnew + ((size_t)l * B + b) * p.Hkv * D + (size_t)g * D;
    const int nq = G * D;
    acquire(cx, nq + 2 * D,
            [&](int i) { return i < nq ? qsrc + i : (i < nq + D ? ksrc + (i - nq) : vsrc + (i - nq - D)); },
            [&](int i, float v) { qs[i] = i < nq ? v * p.inv_sqrt_d : v; });
    cbar(cx, s, seq);
    if (cx.aborted) return;

    const int gi = cx.wave % G, wph = NW / G, sub = cx.wave / G;
    const float* qh = qs + gi * D;
    const uint16_t* Kc = sp.kv + ((((size_t)l * 2 + 0) * B + b) * p.Hkv + g) * (size_t)p.max_seq * D;
    const uint16_t* Vc = sp.kv + ((((size_t)l * 2 + 1) * B + b) * p.Hkv + g) * (size_t)p.max_seq * D;
    const int dpl = D / 64;  // dims per lane in the PV product: lane owns [lane*dpl, lane*dpl + dpl)
    const float ninf = -__builtin_inff();
    float m = ninf, lsum = 0.f, o0 = 0.f, o1 = 0.f;
    const int nkeys = j1 - j0;
    for (int kb = sub; kb * 64 < nkeys; kb += wph) {
        const int j = j0 + kb * 64 + cx.lane;
        const bool valid = j < j1;
        float sc = ninf;
        if (valid) {
            float acc = 0.f;
            if (j < pos) {
                const uint4* kr = (const uint4*)(Kc + (size_t)j * D);
                for (int c = 0; c < D / 8; ++c) {
                    const uint4 w = kr[c];
                    const float4 a = *(const float4*)(qh + c * 8), bq = *(const float4*)(qh + c * 8 + 4);
                    acc += dot8(w, a, bq);
                }
            } else {  // j == pos: the row written by this step
                for (int d = 0; d < D; ++d) acc = fmaf(qh[d], kn[d], acc);
            }
            sc = acc;
        }
        const float mb = wave_max(sc);
        const float mn = fmaxf(m, mb);
        const float e = valid ? __expf(sc - mn) : 0.f;
        const float corr = m == ninf ? 0.f : __expf(m - mn);
        lsum = lsum * corr + wave_sum(e);
        o0 *= corr;
        o1 *= corr;
        m = mn;
        ev[cx.wave * 64 + cx.lane] = e;
        CBAR();
        const int nb = min(64, j1 - (j0 + kb * 64));
        for (int jj = 0; jj < nb; ++jj) {
            const int jk = j0 + kb * 64 + jj;
            const float ej = ev[cx.wave * 64 + jj];
            float v0, v1 = 0.f;
            if (jk < pos) {
                if (dpl == 1) {
                    v0 = bf2f(Vc[(size_t)jk * D + cx.lane]);
                } else {
                    const uint32_t two = *(const uint32_t*)(Vc + (size_t)jk * D + 2 * cx.lane);
                    v0 = bf_lo(two);
                    v1 = bf_hi(two);
                }
            } else {
                v0 = vn[cx.lane * dpl];
                if (dpl == 2) v1 = vn[cx.lane * 2 + 1];
            }
            o0 = fmaf(ej, v0, o0);
            o1 = fmaf(ej, v1, o1);
        }
        CBAR();
    }
    // per-wave state -> LDS, merge per head
    float* my = stt + cx.wave * (D + 2);
    if (cx.lane == 0) {
        my[0] = m;
        my[1] = lsum;
    }
    my[2 + cx.lane * dpl] = o0;
    if (dpl == 2) my[2 + cx.lane * 2 + 1] = o1;
    cbar(cx, s, seq);
    if (sub != 0 || cx.aborted) return;
    float M = ninf;
    for (int w = gi; w < NW; w += G) M = fmaxf(M, stt[w * (D + 2)]);
    float Ls = 0.f, O0 = 0.f, O1 = 0.f;
    if (M != ninf) {
        for (int w = gi; w < NW; w += G) {
            const float* sw = stt + w * (D + 2);
            const float f = sw[0] == ninf ? 0.f : __expf(sw[0] - M);
            Ls = fmaf(sw[1], f, Ls);
            O0 = fmaf(sw[2 + cx.lane * dpl], f, O0);
            if (dpl == 2) O1 = fmaf(sw[2 + cx.lane * 2 + 1], f, O1);
        }
    }
    const int head = g * G + gi;
    uint64_t* out = p.part + ((((size_t)l * B + b) * p.Hq + head) * p.n_split + split) * (D + 2);
    if (cx.lane == 0) {
        st_tag(out + 0, M, cx.epoch);
        st_tag(out + 1, Ls, cx.epoch);
    }
    st_tag(out + 2 + cx.lane * dpl, O0, cx.epoch);
    if (dpl == 2) st_tag(out + 2 + cx.lane * 2 + 1, O1, cx.epoch);
}

// Log-sum-exp merge of the n_split partials of (row b, head):
// out = sum_s o_s e^(m_s - M) / sum_s l_s e^(m_s - M), M = max_s m_s.
__device__ __forceinline__ void op_reduce(Ctx& cx, const Lds& s, uint32_t& seq, const Inst& in, float* xb) {
    const Params& p = *cx.p;
    const int B = p.B, D = p.D, l = in.layer, b = in.a, head = in.b, ns = p.n_split, W = D + 2;
    const uint64_t* src = p.part + (((size_t)l * B + b) * p.Hq + head) * ns * W;
    acquire(cx, ns * W, [&](int i) { return src + i; }, [&](int i, float v) { xb[i] = v; });
    cbar(cx, s, seq);
    if (cx.wave != 0 || cx.aborted) return;
    const float ninf = -__builtin_inff();
    float M = ninf;
    for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, xb[sp * W]);
    const int dpl = D / 64;
    float Ls = 0.f, O0 = 0.f, O1 = 0.f;
    for (int sp = 0; sp < ns; ++sp) {
        const float ms = xb[sp * W];
        if (ms == ninf) continue;
        const float f = __expf(ms - M);
        Ls = fmaf(xb[sp * W + 1], f, Ls);
        O0 = fmaf(xb[sp * W + 2 + cx.lane * dpl], f, O0);
        if (dpl == 2) O1 = fmaf(xb[sp * W + 2 + cx.lane * 2 + 1], f, O1);
    }
    const float inv = 1.0f / Ls;
    uint64_t* out = p.attn + ((size_t)l * B + b) * p.Hq * D + (size_t)head * D;
    st_tag(out + cx.lane * dpl, O0 * inv, cx.epoch);
    if (dpl == 2) st_tag(out + cx.lane * 2 + 1, O1 * inv, cx.epoch);
}

// --------------------------------------------------------------- the kernel --

// stage < 0: run the whole queue (one launch per step); stage >= 0: only that
// stage's instructions (one launch per op and layer).
__global__ void __launch_bounds__(WG_THREADS, 1)
mk_step_kernel(const Params* __restrict__ pp, const int32_t* tokens, const int32_t* positions, uint16_t* kv,
               float* logits, int stage, uint32_t flags) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const Params& p = *pp;
    Ctx cx;
    cx.p = pp;
    cx.cu = blockIdx.x;
    cx.lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    cx.aborted = false;
    cx.pc = 0;
    cx.op = 0;
    cx.epoch = p.epoch[cx.cu] + 1;
    const Lds s = lds_map(smem, p);

    // batch inputs: every workgroup validates them; one bad id stops the step
    Step sp;
    sp.tokens = tokens;
    sp.positions = positions;
    sp.kv = kv;
    sp.logits = logits;
    sp.tok = 0;
    sp.pos = 0;
    {
        int bad = 0;
        uint32_t detail = 0;
        for (int b = 0; b < p.B; ++b) {
            const int t = tokens[b], q = positions[b];
            if (t < 0 || t >= p.V) { bad = 2; detail = (uint32_t)b; }
            else if (q < 0 || q >= p.max_seq) { bad = 3; detail = (uint32_t)b; }
        }
        if (bad) {
            if (threadIdx.x == 0 && cx.cu == 0) {
                cx.wave = 0;
                record_error(cx, (uint32_t)bad, detail);
            }
            return;
        }
        if (cx.lane < p.B) {
            sp.tok = tokens[cx.lane];
            sp.pos = positions[cx.lane];
        }
    }

    const uint32_t qb = p.queue_begin[cx.cu], qlen = p.queue_begin[cx.cu + 1] - qb;
    uint32_t pc0 = 0, pc1 = qlen;
    if (stage >= 0) {
        pc0 = p.stage_pc[(size_t)cx.cu * (p.n_stages + 1) + stage];
        pc1 = p.stage_pc[(size_t)cx.cu * (p.n_stages + 1) + stage + 1];
    }
    if (threadIdx.x < 2 * NW + 4) ((uint32_t*)s.landed)[threadIdx.x] = 0;
    __syncthreads();

    const uint32_t* uoff = p.unit_off + ((size_t)qb + cx.cu) * NW;
    if (wave >= NW) {  // loader
        const int w = wave - NW;
        cx.wave = w;
        loader(cx, s, w, uoff[(size_t)pc0 * NW + w], uoff[(size_t)pc1 * NW + w]);
        return;
    }
    cx.wave = wave;
    Stream st{0, 0};
    uint32_t seq = 0;
    for (uint32_t pc = pc0; pc < pc1 && !cx.aborted; ++pc) {
        const Inst in = p.insts[qb + pc];
        cx.pc = pc;
        cx.op = in.op;
        float* xb = (pc - pc0) & 1 ? s.xbuf[1] : s.xbuf[0];
        switch (in.op) {
        case OP_ATTENTION: op_attention(cx, s, seq, in, xb, sp); break;
        case OP_ATTN_REDUCE: op_reduce(cx, s, seq, in, xb); break;
        default: op_gemv(cx, s, st, seq, in, xb, sp); break;
        }
    }
    if ((flags & KF_BUMP_EPOCH) && wave == 0 && cx.lane == 0) p.epoch[cx.cu] = cx.epoch;
}

// ------------------------------------------------------------ pack kernel --

struct PackRowDev {
    uint32_t mat, row, k0, klen, src_cols, kunits;
    uint64_t dst_unit;
};

// One workgroup per stream row: dst[unit .. unit + kunits) = src row slice, zero padded.
__global__ void __launch_bounds__(256) mk_pack_kernel(const PackRowDev* rows, uint32_t n, const uint16_t* const* mats,
                                                      uint8_t* dst) {
    for (uint32_t r = blockIdx.x; r < n; r += gridDim.x) {
        const PackRowDev pr = rows[r];
        const uint16_t* src = mats[pr.mat] + (size_t)pr.row * pr.src_cols + pr.k0;
        uint16_t* out = (uint16_t*)(dst + pr.dst_unit * (uint64_t)UNIT_BYTES);
        const uint32_t n_el = pr.kunits * UNIT_ELEMS;
        for (uint32_t e = threadIdx.x; e < n_el; e += blockDim.x) out[e] = e < pr.klen ? src[e] : (uint16_t)0;
    }
}

// ------------------------------------------------------------ host launch --

// The whole-step launch waits across workgroups, so it needs every workgroup
// resident at once: a cooperative launch guarantees that (or fails).  Per-op
// launches only read results of earlier launches and use an ordinary launch.
hipError_t launch_step(const Params* dev_params, int ncu, size_t lds_bytes, const int32_t* tokens,
                       const int32_t* positions, void* kv, float* logits, int stage, uint32_t flags,
                       hipStream_t stream) {
    uint16_t* kv16 = (uint16_t*)kv;
    if (stage < 0) {
        void* args[] = {(void*)&dev_params, (void*)&tokens, (void*)&positions, (void*)&kv16, (void*)&logits,
                        (void*)&stage, (void*)&flags};
        return hipLaunchCooperativeKernel((const void*)mk_step_kernel, dim3(ncu), dim3(WG_THREADS), args,
                                          (unsigned)lds_bytes, stream);
    }
    hipLaunchKernelGGL(mk_step_kernel, dim3(ncu), dim3(WG_THREADS), lds_bytes, stream, dev_params, tokens, positions,
                       kv16, logits, stage, flags);
    return hipGetLastError();
}

hipError_t set_step_kernel_lds(size_t lds_bytes) {
    return hipFuncSetAttribute((const void*)mk_step_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
}

hipError_t launch_pack(const void* rows, uint32_t n, const uint16_t* const* mats, uint8_t* dst, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const uint32_t grid = n < 65536 ? n : 65536;
    hipLaunchKernelGGL(mk_pack_kernel, dim3(grid), dim3(256), 0, stream, (const PackRowDev*)rows, n, mats, dst);
    return hipGetLastError();
}

}  // namespace mk
