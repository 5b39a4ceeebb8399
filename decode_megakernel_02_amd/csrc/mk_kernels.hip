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

constexpr int MAXOUT = 16;  // DMA units in flight per loader wave
constexpr int NSERVE = NW / NLOAD;
static_assert(NSERVE == 2, "each loader wave serves two compute waves");

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
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
    case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
    }
}
static_assert(MAXOUT == 16, "wait_vm_le covers 0..15");

// ------------------------------------------------------------ wave context --

struct Ctx {
    const Params* p;
    int cu, wave, lane;
    uint32_t epoch;
    uint32_t pc;       // instruction index in this CU's queue (for error records)
    uint32_t op;
    bool aborted;
    bool prof;         // accumulate cycle counters
    uint64_t cnt[5];   // see mk_get_profile
};

__device__ __forceinline__ uint64_t cycles() { return __builtin_readcyclecounter(); }

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
    const uint64_t t0 = cx.prof ? cycles() : 0;
    seq += NW;
    CBAR();
    if (cx.lane == 0) __hip_atomic_fetch_add(s.bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    uint32_t spins = 0;
    while (lds_ld(s.bar) < seq)
        if (!keep_waiting(cx, spins, 0xBA000000u | seq)) break;
    CBAR();
    if (cx.prof) cx.cnt[3] += cycles() - t0;
}

// ------------------------------------------------------------- loader wave --

// One compute wave's stream as seen by its loader.  Every field is wave
// uniform (scalar registers).
struct LoadStream {
    const uint8_t* src;   // this lane's 16 bytes of unit 0
    uint32_t ring_lds;    // LDS byte address of the ring
    uint32_t n, issued, done, slot, consumed;
    uint32_t a_landed, a_consumed;
};

__device__ __forceinline__ void load_stream_init(const Ctx& cx, const Lds& s, LoadStream& ls, int w, uint32_t ub,
                                                 uint32_t ue) {
    const Params& p = *cx.p;
    // the loaded values are the same in every lane: make that visible to the
    // compiler so the loader's loop state lives in scalar registers
    ub = __builtin_amdgcn_readfirstlane(ub);
    ue = __builtin_amdgcn_readfirstlane(ue);
    const uint64_t base = p.stream_base[cx.cu * NW + w];
    const uint64_t base_u = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(base >> 32)) << 32) |
                            __builtin_amdgcn_readfirstlane((uint32_t)base);
    ls.src = p.wstream + (base_u + (uint64_t)ub * NW) * UNIT_BYTES + cx.lane * 16;
    ls.ring_lds = __builtin_amdgcn_readfirstlane(lds_addr(s.ring + (size_t)w * p.ring_units * UNIT_BYTES));
    ls.n = ue - ub;
    ls.issued = ls.done = ls.slot = ls.consumed = 0;
    ls.a_landed = lds_addr(&s.landed[w]);
    ls.a_consumed = lds_addr(&s.consumed[w]);
}

// issue the stream's next unit if its ring has a free slot (re-reading the
// consumer's count only when the ring looks full)
__device__ __forceinline__ bool load_stream_issue(LoadStream& ls, uint32_t ru) {
    if (ls.issued >= ls.n) return false;
    if (ls.issued >= ls.consumed + ru) {
        ls.consumed = __builtin_amdgcn_readfirstlane(asm_lds_ld(ls.a_consumed));
        if (ls.issued >= ls.consumed + ru) return false;
    }
    __builtin_amdgcn_global_load_lds((const glb_void*)(ls.src + (uint64_t)ls.issued * (NW * UNIT_BYTES)),
                                     (lds_void*)(uintptr_t)(ls.ring_lds + ls.slot * UNIT_BYTES), 16, 0, 0);
    ++ls.issued;
    ls.slot = ls.slot + 1 == ru ? 0 : ls.slot + 1;
    return true;
}

constexpr uint32_t KEEP_IN_FLIGHT = 8;  // units left outstanding when retiring a batch

// Streams the units [ub, ue) of compute waves w0 and w1 into their rings.
// DMA completes in issue order, so a bit FIFO (bit i = stream of the i-th
// oldest outstanding unit) says whose units a vmcnt step retires.  Units are
// retired in batches, keeping KEEP_IN_FLIGHT outstanding while the rings have
// room.  The loader never blocks while DMA is in flight: when both rings are
// full it retires what is outstanding instead, so it cannot wait on a compute
// wave in a cycle.  It runs at raised instruction priority so the compute
// waves' polling cannot starve it of issue slots.
__device__ __forceinline__ void loader(Ctx& cx, const Lds& s, int w0, const uint32_t* uoff, uint32_t pc0,
                                       uint32_t pc1) {
    __builtin_amdgcn_s_setprio(2);
    const uint32_t ru = __builtin_amdgcn_readfirstlane((uint32_t)cx.p->ring_units);
    const int w1 = w0 + 1;
    LoadStream a, b;
    load_stream_init(cx, s, a, w0, uoff[(size_t)pc0 * NW + w0], uoff[(size_t)pc1 * NW + w0]);
    load_stream_init(cx, s, b, w1, uoff[(size_t)pc0 * NW + w1], uoff[(size_t)pc1 * NW + w1]);
    uint32_t fifo = 0, out = 0, spins = 0;
    bool turn_b = false;
    while (a.done < a.n || b.done < b.n) {
        while (out < (uint32_t)MAXOUT) {
            uint32_t sid;
            bool issued;
            if (turn_b) {
                issued = load_stream_issue(b, ru);
                sid = 1;
                if (!issued) { issued = load_stream_issue(a, ru); sid = 0; }
            } else {
                issued = load_stream_issue(a, ru);
                sid = 0;
                if (!issued) { issued = load_stream_issue(b, ru); sid = 1; }
            }
            if (!issued) break;
            fifo |= sid << out;
            ++out;
            turn_b = !turn_b;
        }
        if (out > 0) {
            // retire all but KEEP_IN_FLIGHT units (all of them when nothing more could be issued)
            const bool blocked = out < (uint32_t)MAXOUT;
            const uint32_t keep = blocked ? 0u : KEEP_IN_FLIGHT;
            const uint64_t t0 = cx.prof ? cycles() : 0;
            wait_vm_le(keep);
            if (cx.prof) cx.cnt[1] += cycles() - t0;
            const uint32_t k = out - keep;
            const uint32_t mask = k >= 32 ? 0xffffffffu : (1u << k) - 1u;
            const uint32_t nb = (uint32_t)__builtin_popcount(fifo & mask);
            fifo = k >= 32 ? 0u : fifo >> k;
            out = keep;
            if (k - nb) asm_lds_st(a.a_landed, a.done += k - nb);
            if (nb) asm_lds_st(b.a_landed, b.done += nb);
            if (cx.prof) cx.cnt[3] += k;
            spins = 0;
        } else {
            const uint64_t t0 = cx.prof ? cycles() : 0;
            const bool go_on = keep_waiting(cx, spins, 0x10000000u | (a.done << 12) | b.done);
            if (cx.prof) cx.cnt[2] += cycles() - t0;
            if (!go_on) break;
        }
        if (cx.prof) cx.cnt[4] += 1;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ------------------------------------------------------------ compute side --

struct Stream {  // compute wave's read cursor in its ring
    uint32_t unit;      // units read in this launch
    uint32_t slot;
    uint32_t landed;    // landed count last read from LDS (only ever grows)
    uint32_t released;  // units handed back to the loader
};

// hand the slots read so far back to the loader
__device__ __forceinline__ void ring_release(Ctx& cx, const Lds& s, Stream& st) {
    if (st.released == st.unit) return;
    CBAR();
    lds_st(&s.consumed[cx.wave], st.unit);
    st.released = st.unit;
}
// Next unit of this wave's stream.  Everything already read is released before
// waiting, so the loader always has room to make progress.
__device__ __forceinline__ uint4 ring_take(Ctx& cx, const Lds& s, Stream& st) {
    if (st.unit >= st.landed) {
        ring_release(cx, s, st);
        const uint64_t t0 = cx.prof ? cycles() : 0;
        uint32_t spins = 0;
        while ((st.landed = lds_ld(&s.landed[cx.wave])) <= st.unit)
            if (!keep_waiting(cx, spins, 0x20000000u | st.unit)) break;
        CBAR();
        if (cx.prof) cx.cnt[1] += cycles() - t0;
    }
    if (cx.prof) cx.cnt[4] += 1;
    return *(const uint4*)(s.ring + ((size_t)cx.wave * cx.p->ring_units + st.slot) * UNIT_BYTES + cx.lane * 16);
}
__device__ __forceinline__ void ring_advance(const Ctx& cx, Stream& st) {
    ++st.unit;
    st.slot = st.slot + 1 == (uint32_t)cx.p->ring_units ? 0 : st.slot + 1;
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
// (i, value) to put.  Loads are issued four at a time so latencies overlap.
template <class Addr, class Put>
__device__ __forceinline__ void acquire(Ctx& cx, int n, Addr&& addr, Put&& put) {
    const uint64_t t_begin = cx.prof ? cycles() : 0;
    const int t = cx.wave * 64 + cx.lane;
    constexpr int NT = NW * 64;
    for (int i0 = t; i0 < n; i0 += 4 * NT) {
        uint64_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = i0 + j * NT;
            w[j] = i < n ? ld_tag(addr(i)) : ((uint64_t)cx.epoch << 32);
        }
        uint32_t spins = 0;
        while (true) {
            bool ok = true;
#pragma unroll
            for (int j = 0; j < 4; ++j) ok &= tag_of(w[j]) == cx.epoch;
            if (ok) break;
            if (!keep_waiting(cx, spins, 0x30000000u | (uint32_t)i0)) break;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (tag_of(w[j]) != cx.epoch) w[j] = ld_tag(addr(i0 + j * NT));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = i0 + j * NT;
            if (i < n) put(i, val_of(w[j]));
        }
    }
    if (cx.prof) cx.cnt[2] += cycles() - t_begin;
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

// wait until at least `need` units of this wave's stream have landed;
// everything already read is released first so the loader can progress
__device__ __forceinline__ void ring_wait(Ctx& cx, const Lds& s, Stream& st, uint32_t need) {
    if (st.landed >= need) return;
    ring_release(cx, s, st);
    const uint64_t t0 = cx.prof ? cycles() : 0;
    uint32_t spins = 0;
    while ((st.landed = lds_ld(&s.landed[cx.wave])) < need)
        if (!keep_waiting(cx, spins, 0x20000000u | st.unit)) break;
    CBAR();
    if (cx.prof) cx.cnt[1] += cycles() - t0;
}

// Batch-1 row dot products with this wave's x slice in registers: the KU
// units of a row are read from the ring together and accumulated in KU
// independent chains.
template <int KU>
struct XSlice {
    float4 lo[KU], hi[KU];
};

template <int KU>
__device__ __forceinline__ void load_xslice(const Ctx& cx, const float* xb, int xstride, XSlice<KU>& x) {
    const float4* xr = (const float4*)xb;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
        x.lo[u] = xr[u * 64 + cx.lane];
        x.hi[u] = xr[(xstride >> 3) + u * 64 + cx.lane];
    }
}

template <int KU, int NROWS>
__device__ __forceinline__ void rowgroup_dot_b1(Ctx& cx, const Lds& s, Stream& st, const XSlice<KU>& x, uint32_t ru,
                                                RowOut& out) {
#pragma unroll
    for (int r = 0; r < NROWS; ++r) {
        ring_wait(cx, s, st, st.unit + KU);
        uint4 w[KU];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            uint32_t sl = st.slot + u;
            sl = sl >= ru ? sl - ru : sl;
            w[u] = *(const uint4*)(s.ring + ((size_t)cx.wave * ru + sl) * UNIT_BYTES + cx.lane * 16);
        }
        float acc[KU];
#pragma unroll
        for (int u = 0; u < KU; ++u) acc[u] = dot8(w[u], x.lo[u], x.hi[u]);
        float sum = acc[0];
#pragma unroll
        for (int u = 1; u < KU; ++u) sum += acc[u];
        st.unit += KU;
        st.slot += KU;
        st.slot = st.slot >= ru ? st.slot - ru : st.slot;
        ring_release(cx, s, st);
        if (cx.prof) cx.cnt[4] += KU;
        out.mine[r] = wave_sum(sum);
    }
}

// Dot products of one row-group (NROWS = 1 or 2 rows of ku units each) with x
// for every batch row (x read from LDS); general path for any batch size.
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
            ring_advance(cx, st);
            if ((u & 3) == 3 || u == ku - 1) ring_release(cx, s, st);
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

// KU > 0: batch-1 path with KU units per row (x slice in registers);
// KU == 0: general path.
template <int KU>
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

    XSlice<KU == 0 ? 1 : KU> xs;
    const uint32_t ru = __builtin_amdgcn_readfirstlane((uint32_t)p.ring_units);
    if constexpr (KU > 0) load_xslice<KU>(cx, xb, __builtin_amdgcn_readfirstlane(p.xstride), xs);
    auto dot1 = [&](RowOut& o) {
        if constexpr (KU > 0) rowgroup_dot_b1<KU, 1>(cx, s, st, xs, ru, o);
        else rowgroup_dot<1>(cx, s, st, xb, ku, o);
    };
    auto dot2 = [&](RowOut& o) {
        if constexpr (KU > 0) rowgroup_dot_b1<KU, 2>(cx, s, st, xs, ru, o);
        else rowgroup_dot<2>(cx, s, st, xb, ku, o);
    };

    // ---- this wave's row-groups; lane b < B finishes batch row b
    const int D = p.D, half = D / 2;
    const bool lane_row = cx.lane < B;
    const int b = lane_row ? cx.lane : 0;
    for (uint32_t i = cx.wave; i < in.nrg; i += NW) {
        const uint32_t rg = in.rg0 + i;
        RowOut o;
        switch (in.op) {
        case OP_RMS_QKV_ROPE: {
            dot2(o);
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
            dot1(o);
            if (lane_row) st_tag(p.hmid + ((size_t)l * B + b) * H + rg, hin + o.mine[0], cx.epoch);
            break;
        }
        case OP_RMS_UP_GATE: {
            dot2(o);
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
            dot1(o);
            if (lane_row) {
                float* acc = p.dacc + (size_t)b * H + rg;  // written and read only by this wave's lane b
                const float v = o.mine[0] + (first ? 0.f : *acc);
                if (last) st_tag(p.hout + ((size_t)l * B + b) * H + rg, hm + v, cx.epoch);
                else *acc = v;
            }
            break;
        }
        default: {  // OP_RMS_LM_HEAD
            dot1(o);
            if (lane_row) sp.logits[(size_t)b * p.V + rg] = o.mine[0] * scale;
            break;
        }
        }
        if (cx.aborted) return;
    }
}

// ------------------------------------------------------- attention ops ------

// element i (0..63) of a 64-dim row held as eight packed-bf16 uint4s
__device__ __forceinline__ float bf_elem(const uint4 (&r)[8], int i) {
    const uint4 c = r[i >> 3];
    const uint32_t w = ((i >> 1) & 3) == 0 ? c.x : ((i >> 1) & 3) == 1 ? c.y : ((i >> 1) & 3) == 2 ? c.z : c.w;
    return (i & 1) ? bf_hi(w) : bf_lo(w);
}

// Wave64 reduce-scatter of e * row[d] (d < 64) by recursive halving: afterwards
// lane d holds the sum over lanes of e * row[d].  The first halving step is
// fused with the products so at most 32 values are live; 63 lane exchanges.
__device__ __forceinline__ float pv_reduce_scatter64(const uint4 (&row)[8], float e, int lane) {
    float v[32];
    {
        const bool upper = (lane & 32) != 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int i = h * 16; i < h * 16 + 16; ++i) {
                const float a = e * bf_elem(row, i), b = e * bf_elem(row, i + 32);
                v[i] = (upper ? b : a) + __shfl_xor(upper ? a : b, 32);
            }
            CBAR();
        }
    }
#pragma unroll
    for (int d = 16, m = 32; d >= 1; d >>= 1, m >>= 1) {
        const bool upper = (lane & d) != 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i < m / 2) {
                const float a = v[i], b = v[i + m / 2];
                v[i] = (upper ? b : a) + __shfl_xor(upper ? a : b, d);
            }
        }
    }
    return v[0];
}

// Split-KV partial attention of query heads g*G .. g*G+G-1 of batch row b over
// keys [j0, j1) of split s: writes (m, l, o[D]) with m the max score, l the
// sum of exp(score - m) and o the exp-weighted sum of V rows (unnormalised).
// Waves split the group's heads and 64-key blocks; in a block lane j owns key
// j (its K and V rows, loaded with independent 16-byte loads), and the PV
// product is reduce-scattered so lane d ends with dims d (and d + 64).
template <int D>
__device__ __forceinline__ void op_attention_t(Ctx& cx, const Lds& s, uint32_t& seq, const Inst& in, float* xb,
                                               const Step& sp) {
    constexpr int NH = D / 64;       // 64-dim halves
    const Params& p = *cx.p;
    const int B = p.B, G = p.G, l = in.layer, b = in.a, g = in.b, split = (int)in.rg0;
    const int pos = sp.positions[b];
    const int S = pos + 1;
    const int j0 = (int)((long long)split * S / p.n_split), j1 = (int)((long long)(split + 1) * S / p.n_split);
    float* qs = xb;                  // [G][D], pre-scaled by 1/sqrt(D)
    float* kn = qs + G * D;          // [D] new K row (bf16 values)
    float* vn = kn + D;              // [D] new V row
    float* stt = vn + D;             // [NW][D + 2] per-wave (m, l, o)
    const int gi = cx.wave % G, wph = NW / G, sub = cx.wave / G;
    const uint16_t* Kc = sp.kv + ((((size_t)l * 2 + 0) * B + b) * p.Hkv + g) * (size_t)p.max_seq * D;
    const uint16_t* Vc = sp.kv + ((((size_t)l * 2 + 1) * B + b) * p.Hkv + g) * (size_t)p.max_seq * D;
    const int nkeys = j1 - j0;

    // K rows written by earlier steps do not depend on this step: load the
    // first block's first 64 dims before waiting for q.  Rows are handled in
    // 64-dim halves (eight 16-byte chunks) to bound register use.
    uint4 kr[8], vr[8];
    auto load_half = [&](uint4 (&r)[8], const uint16_t* base, int kb, int h) {
        const int j = j0 + kb * 64 + cx.lane;
        const bool old = j < j1 && j < pos;
        const uint4* src = (const uint4*)(base + (size_t)(old ? j : 0) * D + h * 64);
#pragma unroll
        for (int c = 0; c < 8; ++c) r[c] = old ? src[c] : make_uint4(0, 0, 0, 0);
    };
    auto pack_lds = [&](uint4 (&r)[8], const float* row) {  // exact: the values are bf16
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float* v = row + c * 8;
            r[c] = make_uint4((uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16),
                              (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16),
                              (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16),
                              (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16));
        }
    };
    if (sub * 64 < nkeys) load_half(kr, Kc, sub, 0);

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

    const float* qh = qs + gi * D;
    const float ninf = -__builtin_inff();
    float m = ninf, lsum = 0.f, o[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) o[h] = 0.f;
    for (int kb = sub; kb * 64 < nkeys; kb += wph) {
        const int j = j0 + kb * 64 + cx.lane;
        const bool valid = j < j1;
        const bool is_new = valid && j == pos;  // the row this step appended: from LDS
        float acc = 0.f;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            CBAR();  // keeps the two halves' loads apart (register budget)
            if (kb != sub || h != 0) load_half(kr, Kc, kb, h);
            if (is_new) pack_lds(kr, kn + h * 64);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float4 a = *(const float4*)(qh + h * 64 + c * 8), bq = *(const float4*)(qh + h * 64 + c * 8 + 4);
                acc += dot8(kr[c], a, bq);
            }
        }
        const float sc = valid ? acc : ninf;
        const float mn = fmaxf(m, wave_max(sc));
        const float e = valid ? __expf(sc - mn) : 0.f;
        const float corr = m == ninf ? 0.f : __expf(m - mn);
        lsum = lsum * corr + wave_sum(e);
        m = mn;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            CBAR();
            load_half(vr, Vc, kb, h);
            if (is_new) pack_lds(vr, vn + h * 64);
            o[h] = o[h] * corr + pv_reduce_scatter64(vr, e, cx.lane);
        }
    }
    // per-wave state -> LDS, merge the waves of each head
    float* my = stt + cx.wave * (D + 2);
    if (cx.lane == 0) {
        my[0] = m;
        my[1] = lsum;
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) my[2 + h * 64 + cx.lane] = o[h];
    cbar(cx, s, seq);
    if (sub != 0 || cx.aborted) return;
    float M = ninf;
    for (int w = gi; w < NW; w += G) M = fmaxf(M, stt[w * (D + 2)]);
    float Ls = 0.f, O[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) O[h] = 0.f;
    if (M != ninf) {
        for (int w = gi; w < NW; w += G) {
            const float* sw = stt + w * (D + 2);
            const float f = sw[0] == ninf ? 0.f : __expf(sw[0] - M);
            Ls = fmaf(sw[1], f, Ls);
#pragma unroll
            for (int h = 0; h < NH; ++h) O[h] = fmaf(sw[2 + h * 64 + cx.lane], f, O[h]);
        }
    }
    const int head = g * G + gi;
    uint64_t* out = p.part + ((((size_t)l * B + b) * p.Hq + head) * p.n_split + split) * (D + 2);
    if (cx.lane == 0) {
        st_tag(out + 0, M, cx.epoch);
        st_tag(out + 1, Ls, cx.epoch);
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) st_tag(out + 2 + h * 64 + cx.lane, O[h], cx.epoch);
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
    const int nh = D / 64;  // lane owns dims lane (and lane + 64)
    float Ls = 0.f, O0 = 0.f, O1 = 0.f;
    for (int sp = 0; sp < ns; ++sp) {
        const float ms = xb[sp * W];
        if (ms == ninf) continue;
        const float f = __expf(ms - M);
        Ls = fmaf(xb[sp * W + 1], f, Ls);
        O0 = fmaf(xb[sp * W + 2 + cx.lane], f, O0);
        if (nh == 2) O1 = fmaf(xb[sp * W + 2 + 64 + cx.lane], f, O1);
    }
    const float inv = 1.0f / Ls;
    uint64_t* out = p.attn + ((size_t)l * B + b) * p.Hq * D + (size_t)head * D;
    st_tag(out + cx.lane, O0 * inv, cx.epoch);
    if (nh == 2) st_tag(out + 64 + cx.lane, O1 * inv, cx.epoch);
}

// --------------------------------------------------------------- the kernel --

// stage < 0: run the whole queue (one launch per step); stage >= 0: only that
// stage's instructions (one launch per op and layer).  One instantiation per
// head size.
template <int HEAD_DIM>
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
    cx.prof = p.prof != nullptr;
    for (int k = 0; k < 5; ++k) cx.cnt[k] = 0;
    const uint64_t t_kernel = cx.prof ? cycles() : 0;
    auto flush_prof = [&](int wave_slot) {
        if (cx.prof && cx.lane == 0) {
            uint64_t* o = p.prof + ((size_t)cx.cu * (NW + NLOAD) + wave_slot) * PROF_SLOTS;
            o[0] = cycles() - t_kernel;
            for (int k = 1; k < 5; ++k) o[k] = cx.cnt[k];
        }
    };
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
    if (wave >= NW) {  // loader of compute waves 2i and 2i+1
        const int w0 = (wave - NW) * NSERVE;
        cx.wave = wave;
        loader(cx, s, w0, uoff, pc0, pc1);
        flush_prof(wave);
        return;
    }
    cx.wave = wave;
    Stream st{0, 0, 0, 0};
    uint32_t seq = 0;
    for (uint32_t pc = pc0; pc < pc1 && !cx.aborted; ++pc) {
        const Inst in = p.insts[qb + pc];
        cx.pc = pc;
        cx.op = in.op;
        float* xb = (pc - pc0) & 1 ? s.xbuf[1] : s.xbuf[0];
        switch (in.op) {
        case OP_ATTENTION: op_attention_t<HEAD_DIM>(cx, s, seq, in, xb, sp); break;
        case OP_ATTN_REDUCE: op_reduce(cx, s, seq, in, xb); break;
        default: {
            const int ku = in.op == OP_O_PROJ_RES ? p.ku_q : in.op == OP_DOWN_RES ? p.ku_f : p.ku_h;
            if (p.B != 1) op_gemv<0>(cx, s, st, seq, in, xb, sp);
            else if (ku == 4) op_gemv<4>(cx, s, st, seq, in, xb, sp);
            else if (ku == 2) op_gemv<2>(cx, s, st, seq, in, xb, sp);
            else op_gemv<0>(cx, s, st, seq, in, xb, sp);
            break;
        }
        }
    }
    flush_prof(wave);
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
        const uint32_t n_el = pr.kunits * UNIT_ELEMS;
        for (uint32_t e = threadIdx.x; e < n_el; e += blockDim.x) {
            // element e lies in the row's unit e / 512, and consecutive units of a
            // stream are NW units apart in the packed buffer
            uint16_t* out = (uint16_t*)(dst + (pr.dst_unit + (uint64_t)(e / UNIT_ELEMS) * NW) * UNIT_BYTES);
            out[e % UNIT_ELEMS] = e < pr.klen ? src[e] : (uint16_t)0;
        }
    }
}

// ------------------------------------------------------------ host launch --

// The whole-step launch waits across workgroups, so it needs every workgroup
// resident at once: a cooperative launch guarantees that (or fails).  Per-op
// launches only read results of earlier launches and use an ordinary launch.
hipError_t launch_step(const Params* dev_params, int head_dim, int ncu, size_t lds_bytes, const int32_t* tokens,
                       const int32_t* positions, void* kv, float* logits, int stage, uint32_t flags,
                       hipStream_t stream) {
    uint16_t* kv16 = (uint16_t*)kv;
    const void* fn = head_dim == 64 ? (const void*)mk_step_kernel<64> : (const void*)mk_step_kernel<128>;
    void* args[] = {(void*)&dev_params, (void*)&tokens, (void*)&positions, (void*)&kv16, (void*)&logits,
                    (void*)&stage, (void*)&flags};
    if (stage < 0)
        return hipLaunchCooperativeKernel(fn, dim3(ncu), dim3(WG_THREADS), args, (unsigned)lds_bytes, stream);
    return hipLaunchKernel(fn, dim3(ncu), dim3(WG_THREADS), args, lds_bytes, stream);
}

hipError_t set_step_kernel_lds(size_t lds_bytes) {
    hipError_t e = hipFuncSetAttribute((const void*)mk_step_kernel<64>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds_bytes);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute((const void*)mk_step_kernel<128>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds_bytes);
}

hipError_t launch_pack(const void* rows, uint32_t n, const uint16_t* const* mats, uint8_t* dst, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const uint32_t grid = n < 65536 ? n : 65536;
    hipLaunchKernelGGL(mk_pack_kernel, dim3(grid), dim3(256), 0, stream, (const PackRowDev*)rows, n, mats, dst);
    return hipGetLastError();
}

}  // namespace mk
