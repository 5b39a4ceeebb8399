// Device code for gfx950 (MI355X): the persistent decode interpreter, its op
// bodies, and the weight-pack kernel.
//
// One workgroup per CU runs 8 compute waves, 3 weight-loader waves and 1
// gather wave.  Loader wave i streams the packed weights of compute waves i,
// i + 3 and i + 6 (each a byte stream laid out at load time in exactly the
// order that wave consumes it) from HBM into the waves' private LDS rings with
// global->LDS DMA, ahead of the dependency waits: weights never
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

// This file is compiled twice: the step kernels for batch-1 handles (MK_BATCHED_TU 0, which also
// holds every other kernel and the host entry points) and for handles with several batch rows
// (MK_BATCHED_TU 1).  Each build then carries only the code its batch size takes: the batch-1
// step keeps none of the 2..8-row dot products, the compute waves' own-row gather or the paired
// LM-head rows, and stays within its register budget.
#ifndef MK_BATCHED_TU
#define MK_BATCHED_TU 0
#endif
constexpr bool TU_BATCHED = MK_BATCHED_TU != 0;

// Explicit address spaces: the compiler otherwise emits flat instructions for
// pointers it cannot trace, and a flat access to LDS is routed through the
// vector-memory path, where it queues behind the loader's DMA.
#define LDS __attribute__((address_space(3)))
#define GLB __attribute__((address_space(1)))
typedef LDS void lds_void;
typedef GLB void glb_void;
// Kernel parameters are read through the constant address space: they never
// change during a launch, and no LDS or global store can alias them, so the
// compiler keeps loaded fields instead of re-reading them after every store.
typedef const __attribute__((address_space(4))) Params CParams;
// The instruction queues never change during a launch either: read through the
// constant address space they become scalar loads, which are waited for with
// the LDS/scalar counter instead of the vector-memory counter (a vector load
// would make the wave wait for its own outstanding stores as well).
#define CONST_AS __attribute__((address_space(4)))

template <class T>
__device__ __forceinline__ T gld(const T* p) {
    return *(const GLB T*)p;
}
// vector loads through native clang vector types (HIP's vector structs copy
// through generic references, which turns them back into flat accesses)
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 gld_u4(const void* p) {
    const u32x4 v = *(const GLB u32x4*)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 lds_u4(const LDS void* p) {
    const u32x4 v = *(const LDS u32x4*)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 lds_f4(const LDS float* p) {
    const f32x4 v = *(const LDS f32x4*)p;
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float2 gld_f2(const float* p) {
    const u32x2 v = *(const GLB u32x2*)p;
    return make_float2(__uint_as_float(v.x), __uint_as_float(v.y));
}
// Waits until none of this wave's vector-memory operations is outstanding, as
// an instruction the compiler's wait-insertion pass sees (so it stops tracking
// earlier loads).  gfx9 encoding: vmcnt 0, expcnt 7, lgkmcnt 15.
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// A load whose value is waited for on the spot.  Used on rarely taken paths of
// the compute waves: a load left outstanding across a branch join makes the
// compiler wait for the whole vector-memory counter at a later register
// reuse, and on gfx9 that counter includes the wave's own stores, whose
// acknowledgement from the coherent memory level takes microseconds.
template <class T>
__device__ __forceinline__ T gld_now(const T* p) {
    const T v = gld(p);
    vm_drain();
    return v;
}
template <class T>
__device__ __forceinline__ void gst(T* p, T v) {
    *(GLB T*)p = v;
}

#define CBAR() asm volatile("" ::: "memory")

constexpr int NGATHER = 1;  // gather waves
constexpr int NWL = 1;      // weight loader waves
static_assert(NLOAD == NWL + NGATHER, "one loader wave and one gather wave");

// ------------------------------------------------------------- primitives --

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// float -> bf16 bits, round to nearest even
// (branch free: it runs in single active lanes of a wave)
__device__ __forceinline__ uint16_t f2bf(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t q = (u >> 16) | 0x40u;  // NaN: keep it a quiet NaN
    return (uint16_t)((u & 0x7fffffffu) > 0x7f800000u ? q : r);
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
    __hip_atomic_store((GLB uint64_t*)p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tag(const uint64_t* p) {
    return __hip_atomic_load((GLB uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t tag_of(uint64_t w) { return (uint32_t)(w >> 32); }
__device__ __forceinline__ float val_of(uint64_t w) { return __uint_as_float((uint32_t)w); }

// LDS sync words between waves of one workgroup.  LDS requests of one wave
// complete in order, so a data write followed by a flag write is observed in
// that order by any wave that reads the flag and then the data.
__device__ __forceinline__ uint32_t lds_ld(const LDS uint32_t* p) {
    return __hip_atomic_load((LDS uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(LDS uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// The loader wave issues LDS DMA; the compiler would guard its own LDS
// accesses with vmcnt(0) waits (the DMA may alias them), so the loader touches
// its sync words through inline asm instead.
__device__ __forceinline__ uint32_t lds_addr(const lds_void* p) { return (uint32_t)(uintptr_t)p; }
__device__ __forceinline__ uint32_t asm_lds_ld(uint32_t a) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
    return v;
}
__device__ __forceinline__ void asm_lds_st(uint32_t a, uint32_t v) {
    asm volatile("ds_write_b32 %0, %1" ::"v"(a), "v"(v) : "memory");
}
__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Smallest of the 8 words at a (16-byte aligned): two 16-byte reads and one wait, inside the
// block (the outputs are early-clobber: the second read still needs the address register)
__device__ __forceinline__ uint32_t asm_lds_min8(uint32_t a) {
    u32x4 v0, v1;
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:16\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v0), "=&v"(v1)
                 : "v"(a)
                 : "memory");
    const uint32_t m0 = min(min(v0.x, v0.y), min(v0.z, v0.w)), m1 = min(min(v1.x, v1.y), min(v1.z, v1.w));
    return min(m0, m1);
}

// ------------------------------------------------------------ wave context --

struct Ctx {
    CParams* p;
    int cu, wave, lane;
    uint32_t epoch;
    uint32_t pc;       // instruction index in this CU's queue (for error records)
    uint32_t slot;     // buffer set of the current instruction's staged inputs
    uint32_t op;
    bool aborted;
    bool resident;     // one launch for the whole step: the CU's residual rows stay in LDS between ops
    bool prof;         // accumulate cycle counters
    bool trace;        // write timeline records
    uint64_t t_acq;    // real time at which the current instruction's cross-CU inputs were loaded
    uint64_t t_in;     // real time at which the current instruction's inputs were ready
    uint64_t t_mid;    // real time at which the main loop ended
    uint64_t t_ring;   // real-time ticks spent waiting for weight units in the current instruction
    uint64_t cnt[8];   // see mk_get_profile
};
constexpr uint32_t GREEDY_NONE = 0xffffffffu;
// Fused greedy: a (value, row) candidate as one 64-bit key whose unsigned order is the selection
// order: the float's bits mapped to an order-preserving unsigned integer (-0 taken as +0, so that
// equal values tie) above the row's complement (the lower row wins a tie).  0 is below every
// key: no candidate.
__device__ __forceinline__ uint64_t greedy_key(float v, uint32_t row) {
    uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint64_t)(0xffffffffu - row);
}
__device__ __forceinline__ void greedy_unkey(uint64_t k, float& v, uint32_t& row) {
    if (k == 0) {
        v = -__builtin_inff();
        row = GREEDY_NONE;
        return;
    }
    uint32_t u = (uint32_t)(k >> 32);
    u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
    v = __uint_as_float(u);
    row = 0xffffffffu - (uint32_t)k;
}

__device__ __forceinline__ uint64_t cycles() { return __builtin_readcyclecounter(); }
// constant-rate (100 MHz) clock shared by all CUs
__device__ __forceinline__ uint64_t rtime() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ void mark_inputs(Ctx& cx) {
    if (cx.trace) cx.t_in = rtime();
}
__device__ __forceinline__ void mark_acquired(Ctx& cx) {
    if (cx.trace) cx.t_acq = rtime();
}
__device__ __forceinline__ void mark_mid(Ctx& cx) {
    if (cx.trace) cx.t_mid = rtime();
}

__device__ __forceinline__ bool abort_flag(CParams* p) {
    return __hip_atomic_load((GLB uint32_t*)&p->error[7], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}
__device__ __forceinline__ void record_error_rec(uint32_t* e, uint32_t code, uint32_t cu, uint32_t pc, uint32_t op,
                                             uint32_t wave, uint32_t detail) {
    GLB uint32_t* g = (GLB uint32_t*)e;
    uint32_t expected = 0u;
    if (__hip_atomic_compare_exchange_strong(g, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT)) {
        g[1] = cu;
        g[2] = pc;
        g[3] = op;
        g[4] = wave;
        g[5] = detail;
    }
    __hip_atomic_store((GLB uint32_t*)&e[7], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void record_error(Ctx& cx, uint32_t code, uint32_t detail) {
    record_error_rec(cx.p->error, code, (uint32_t)cx.cu, cx.pc, cx.op, (uint32_t)cx.wave, detail);
    cx.aborted = true;
}
// one iteration of a bounded wait; returns false once the wait must give up
// Every wait loop polls on wave-uniform values (scalar branches) and sleeps
// between polls: spinning waves would otherwise take most of the CU's scalar
// issue slots away from the waves doing the work.
__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ bool any_lane(bool c) { return __builtin_amdgcn_ballot_w64(c) != 0; }

#ifndef MK_SLEEP
#define MK_SLEEP 1
#endif
template <int SLEEP = MK_SLEEP>
__device__ __forceinline__ bool keep_waiting(Ctx& cx, uint32_t& spins, uint32_t detail) {
    if (uni(cx.aborted)) return false;
    ++spins;
    if ((spins & 1023u) == 0u && abort_flag(cx.p)) {
        cx.aborted = true;
        return false;
    }
    if (spins > cx.p->spin_limit) {
        record_error(cx, 1u, detail);
        return false;
    }
    __builtin_amdgcn_s_sleep(SLEEP);
    return true;
}

// ---------------------------------------------------------------- LDS map --

// counters, ss, the greedy keys and the last-CU flag, zeroed at launch
constexpr int SYNC_WORDS = 3 * NW + 4 + MAX_SLOTS * MAX_BATCH + 2 * MAX_BATCH + 1;
static_assert(SYNC_WORDS * 4 <= 512, "the sync words fit the 512-byte sync area");
static_assert((3 * NW + 4 + MAX_SLOTS * MAX_BATCH) % 2 == 0, "the greedy keys are 8-byte aligned");

struct Lds {
    LDS uint8_t* ring;      // [NW][ring_units][1024]
    LDS float* xbuf0;       // nslot x buffers of xbuf_bytes each, back to back
    LDS uint32_t* landed;   // [0]: unit-rows landed in every compute wave's ring ([1 .. NW) unused)
    LDS uint32_t* consumed; // [NW] units consumed
    LDS uint32_t* bar;      // compute-wave barrier counter
    LDS uint32_t* ready;    // [MAX_SLOTS] r + 1 once instruction r's inputs are staged in buffer set r % nslot
    LDS uint32_t* done;     // [NW] instructions each compute wave has finished
    LDS float* ss;          // [MAX_SLOTS][MAX_BATCH] sum of squares of each x buffer's raw input rows
    LDS uint64_t* gkey;     // [MAX_BATCH] fused greedy: the CU's best LM-head row per batch row (greedy_key)
    LDS uint32_t* glast;    // fused greedy: 1 in the CU that merges every CU's rows
    LDS float* side0;       // nslot side buffers (side_floats each): epilogue inputs staged with x buffer i
    LDS float* rope;        // [B][D] (cos, sin) pairs of the step's positions, loaded once per launch
    LDS float* res;         // [B][res_stride] the CU's residual rows (O and down-projection tile)
};
__device__ __forceinline__ Lds lds_map(LDS uint8_t* smem, CParams& p) {
    Lds m;
    m.ring = smem;
    size_t off = (size_t)NW * p.ring_units * UNIT_BYTES;
    m.xbuf0 = (LDS float*)(smem + off);
    LDS uint32_t* sync = (LDS uint32_t*)(smem + off + (size_t)p.nslot * p.xbuf_bytes);
    m.landed = sync;
    m.consumed = sync + NW;
    m.bar = sync + 2 * NW;
    m.ready = sync + 2 * NW + 1;
    m.done = sync + 2 * NW + 4;
    m.ss = (LDS float*)(sync + 3 * NW + 4);
    m.gkey = (LDS uint64_t*)(sync + 3 * NW + 4 + MAX_SLOTS * MAX_BATCH);
    m.glast = sync + 3 * NW + 4 + MAX_SLOTS * MAX_BATCH + 2 * MAX_BATCH;
    m.side0 = (LDS float*)(smem + off + (size_t)p.nslot * p.xbuf_bytes + 512);
    m.rope = m.side0 + (size_t)p.nslot * p.side_floats;
    m.res = m.rope + (size_t)p.B * p.D;
    return m;
}
// buffer set `slot` of the staged inputs
__device__ __forceinline__ LDS float* xslot(const Lds& s, CParams& p, uint32_t slot) {
    return s.xbuf0 + slot * (uint32_t)(p.xbuf_bytes >> 2);
}
__device__ __forceinline__ LDS float* sslot(const Lds& s, CParams& p, uint32_t slot) {
    return s.side0 + slot * (uint32_t)p.side_floats;
}

// barrier among the NW compute waves (loader waves never join it)
__device__ __forceinline__ void cbar(Ctx& cx, const Lds& s, uint32_t& seq) {
    const uint64_t t0 = cx.prof ? cycles() : 0;
    seq += NW;
    CBAR();
    uint32_t old = 0;
    if (cx.lane == 0) old = __hip_atomic_fetch_add(s.bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (uni(old) + 1u == seq) {
        // last to arrive: wake the waves sleeping in this barrier
        asm volatile("s_wakeup" ::: "memory");
        if (cx.prof) cx.cnt[7] += 1;
    } else {
        uint32_t spins = 0;
        while (uni(lds_ld(s.bar)) < seq)
            if (!keep_waiting<4>(cx, spins, 0xBA000000u | seq)) break;
        if (cx.prof) cx.cnt[6] += spins;
    }
    if (cx.prof) cx.cnt[5] += 1;
    CBAR();
    if (cx.prof) cx.cnt[3] += cycles() - t0;
}

// ------------------------------------------------------------- loader wave --

// One loader wave streams the weights of all NW compute waves.  Unit u of
// compute wave w's stream is packed at stream_base[cu * NW + w] + u * NW.
// The loader walks the CU's instructions in queue order and issues each GEMV
// instruction's units as unit-rows: row j holds unit j of the instruction for
// every compute wave, DMA'd into that wave's ring slot (row index) % ring_units.
// An instruction has as many rows as the wave with the most units in it
// needs (field b of the instruction); a wave with fewer units gets a spare
// unit (any resident 1 KiB of the packed buffer) in the rest of its rows and
// skips them.  So row r maps to the same instruction in every ring, one
// `landed` counter (rows fully arrived) serves every wave, and a row is issued
// only when every ring has its slot free (each compute wave publishes how many
// rows it has consumed).  Weights never depend on activations, so the loader
// runs ahead across instruction and layer boundaries as far as the rings
// allow (the page "Megakernels: Deleting the Kernel Boundary to Win Back
// Microseconds", section "Correctness without the free barrier": the next
// instruction's loads start early).  Its loop costs a few scalar instructions
// per unit: it shares a SIMD with compute waves at raised priority, so every
// instruction it spends is taken from them.
#ifndef MK_LOADER_PRIO
#define MK_LOADER_PRIO 2
#endif
#ifndef MK_LOADER_SLEEP
#define MK_LOADER_SLEEP 1
#endif
#ifndef MK_LD_ROWS
#define MK_LD_ROWS 7
#endif
#ifndef MK_LD_KEEP
#define MK_LD_KEEP 2
#endif
constexpr uint32_t LD_ROWS = MK_LD_ROWS;  // unit-rows in flight (NW DMAs each; vmcnt counts at most 63)
constexpr uint32_t LD_KEEP = MK_LD_KEEP;  // unit-rows left in flight when retiring
static_assert(LD_ROWS * NW <= 63 && LD_KEEP < LD_ROWS, "DMA accounting");
// The weights are read once per step: the DMA is non-temporal, so the stream
// does not evict the code, queue and parameter lines the waves keep reusing
// from L2 (measured: 16 us of a 900 us step at the 1B workload).
constexpr int CPOL_NT = 2;
// s_waitcnt immediate (gfx9 layout) that waits for vmcnt <= n only: vmcnt bits 3:0 and 15:14,
// expcnt 6:4 and lgkmcnt 11:8 at their maxima
constexpr int vmcnt_imm(int n) { return ((n >> 4) << 14) | 0xF00 | 0x70 | (n & 15); }
static_assert(vmcnt_imm(0) == 0x0F70, "matches the encoding of vm_drain");

// uoff: the instruction boundaries' unit offsets, read through the constant address space: as
// scalar loads they are waited for with the LDS/scalar counter, where a vector load would wait
// for every DMA in flight (the vector-memory counter covers them all).
__device__ __forceinline__ void loader(Ctx& cx, const Lds& s, const CONST_AS uint32_t* uoff, uint32_t pc0,
                                       uint32_t pc1) {
    __builtin_amdgcn_s_setprio(MK_LOADER_PRIO);
    CParams& p = *cx.p;
    const uint32_t ru = uni((uint32_t)p.ring_units);
    const uint8_t* base[NW];  // wave-uniform: unit 0 of compute wave w's stream
    uint32_t cur[NW];         // wave w's first unit of the instruction being streamed
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint64_t b = p.stream_base[cx.cu * NW + w];
        const uint64_t bu = ((uint64_t)uni((uint32_t)(b >> 32)) << 32) | uni((uint32_t)b);
        base[w] = p.wstream + bu * UNIT_BYTES;
        cur[w] = uni(uoff[(size_t)pc0 * NW + w]);
    }
    // spare source of padding rows: unit 0 of the CU's region (it exists whenever a row is issued)
    const uint8_t* spare = base[0];
    const uint32_t voff = (uint32_t)cx.lane * 16;  // this lane's 16 bytes of a unit
    const uint32_t ring0 = uni(lds_addr(s.ring));
    const uint32_t a_landed = uni(lds_addr(&s.landed[0]));
    uint32_t u = 0, slot = 0, published = 0;
    uint32_t room = ru;  // rows below `room` have a free slot in every ring (nothing consumed yet)
    uint32_t spins = 0;
    bool stop = false;
    auto publish = [&](uint32_t v) {
        published = v;
        asm_lds_st(a_landed, v);
    };
    for (uint32_t pc = pc0; pc < pc1 && !stop; ++pc) {
        uint32_t nxt[NW], rows = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            nxt[w] = uni(uoff[(size_t)(pc + 1) * NW + w]);
            rows = nxt[w] - cur[w] > rows ? nxt[w] - cur[w] : rows;
        }
        for (uint32_t j = 0; j < rows;) {
            if (u >= room) {
                static_assert(NW == 8, "eight consumed counters, read as two 16-byte words");
                room = uni(asm_lds_min8(lds_addr(&s.consumed[0]))) + ru;
                if (u >= room) {
                    const uint64_t t0 = cx.prof ? cycles() : 0;
                    if (published < u) {  // hand over what is in flight before waiting on the consumers
                        wait_vm_all();
                        publish(u);
                    } else if (!keep_waiting<MK_LOADER_SLEEP>(cx, spins, 0x10000000u | u)) {
                        stop = true;
                        break;
                    }
                    if (cx.prof) cx.cnt[2] += cycles() - t0;
                    continue;
                }
                spins = 0;
            }
            const uint32_t dst = ring0 + slot * UNIT_BYTES;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const uint32_t unit = cur[w] + j;
                const uint8_t* src = unit < nxt[w] ? base[w] + (size_t)unit * (NW * UNIT_BYTES) : spare;
                __builtin_amdgcn_global_load_lds((const glb_void*)(src + voff),
                                                 (lds_void*)(uintptr_t)(dst + (uint32_t)w * ru * UNIT_BYTES), 16, 0,
                                                 CPOL_NT);
            }
            slot = slot + 1 == ru ? 0 : slot + 1;
            ++u;
            ++j;
            if (cx.prof) {
                cx.cnt[3] += NW;
                cx.cnt[4] += 1;
            }
            if (u - published >= LD_ROWS) {  // retire all but the LD_KEEP newest rows
                const uint64_t t0 = cx.prof ? cycles() : 0;
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(LD_KEEP * NW));
                publish(u - LD_KEEP);
                if (cx.prof) cx.cnt[1] += cycles() - t0;
            }
        }
#pragma unroll
        for (int w = 0; w < NW; ++w) cur[w] = nxt[w];
    }
    wait_vm_all();
    publish(u);
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
        const uint64_t r0 = cx.trace ? rtime() : 0;
        uint32_t spins = 0;
        while ((st.landed = uni(lds_ld(&s.landed[0]))) <= st.unit)
            if (!keep_waiting(cx, spins, 0x20000000u | st.unit)) break;
        CBAR();
        if (cx.prof) cx.cnt[1] += cycles() - t0;
        if (cx.trace) cx.t_ring += rtime() - r0;
    }
    if (cx.prof) cx.cnt[4] += 1;
    return lds_u4(s.ring + ((size_t)cx.wave * cx.p->ring_units + st.slot) * UNIT_BYTES + cx.lane * 16);
}
__device__ __forceinline__ void ring_advance(const Ctx& cx, Stream& st) {
    ++st.unit;
    st.slot = st.slot + 1 == (uint32_t)cx.p->ring_units ? 0 : st.slot + 1;
}

// x buffer layout per batch row: [half][chunk][4] with element k in half
// (k % 8) / 4, chunk k / 8, position k % 4, so a lane's 8 elements of one unit
// are two 16-byte reads at consecutive addresses across lanes.
// xs = floats per batch row.  For k0 a multiple of 8, xidx(k0 + k) = xidx(k) + k0 / 2.
__device__ __forceinline__ int xidx(int xs, int b, int k) {
    return b * xs + ((k & 4) ? (xs >> 1) : 0) + (k >> 3) * 4 + (k & 3);
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

// One unit of FP8 codes: lane c holds the 16 codes of elements 16c .. 16c+15 of
// the unit, i.e. x chunks 2c (a0: elements 0-3, b0: 4-7) and 2c+1 (a1, b1).
// The conversion instruction decodes OCP E4M3 (checked against the format
// table on this device); the row scale is applied to the row sum.
__device__ __forceinline__ float dot16_fp8(const uint4 w, const float4 a0, const float4 b0, const float4 a1,
                                           const float4 b1) {
    const auto c0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false), c1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
    const auto c2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false), c3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
    const auto c4 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.z, false), c5 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.z, true);
    const auto c6 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.w, false), c7 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.w, true);
    // four independent chains of four (a single chain of sixteen is latency-bound)
    float s0 = c0[0] * a0.x, s1 = c2[0] * b0.x, s2 = c4[0] * a1.x, s3 = c6[0] * b1.x;
    s0 = fmaf(c0[1], a0.y, s0);
    s1 = fmaf(c2[1], b0.y, s1);
    s2 = fmaf(c4[1], a1.y, s2);
    s3 = fmaf(c6[1], b1.y, s3);
    s0 = fmaf(c1[0], a0.z, s0);
    s1 = fmaf(c3[0], b0.z, s1);
    s2 = fmaf(c5[0], a1.z, s2);
    s3 = fmaf(c7[0], b1.z, s3);
    s0 = fmaf(c1[1], a0.w, s0);
    s1 = fmaf(c3[1], b0.w, s1);
    s2 = fmaf(c5[1], a1.w, s2);
    s3 = fmaf(c7[1], b1.w, s3);
    return (s0 + s1) + (s2 + s3);
}

// Poll a single tagged word (epilogue inputs that were produced long before).
__device__ __forceinline__ float wait_word(Ctx& cx, const uint64_t* p) {
    uint64_t w = ld_tag(p);
    uint32_t spins = 0;
    while (any_lane(tag_of(w) != cx.epoch)) {
        if (!keep_waiting(cx, spins, 0x40000000u)) break;
        if (tag_of(w) != cx.epoch) w = ld_tag(p);
    }
    vm_drain();  // leaves no load tracked past this (rarely taken) path
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
    const uint64_t r0 = cx.trace ? rtime() : 0;
    uint32_t spins = 0;
    while ((st.landed = uni(lds_ld(&s.landed[0]))) < need)
        if (!keep_waiting(cx, spins, 0x20000000u | st.unit)) break;
    CBAR();
    if (cx.prof) cx.cnt[1] += cycles() - t0;
    if (cx.trace) cx.t_ring += rtime() - r0;
}

// Ablation build: pass over n units of this wave's stream without reading them, a quarter
// ring at a time (the granularity of the dot products, so the loader keeps streaming instead
// of refilling an emptied ring; everything read is released before each wait); the loader
// still streams them.
__device__ __forceinline__ void ring_skip(Ctx& cx, const Lds& s, Stream& st, uint32_t n) {
    const uint32_t ru = uni((uint32_t)cx.p->ring_units), q = ru / 4 > 0 ? ru / 4 : 1;
    while (n > 0 && !cx.aborted) {
        const uint32_t c = n < q ? n : q;
        ring_wait(cx, s, st, st.unit + c);
        st.unit += c;
        st.slot = (st.slot + c) % ru;
        ring_release(cx, s, st);
        n -= c;
    }
}

// Batch-1 row dot products with this wave's x slice in registers: the KU
// units of a row are read from the ring together and accumulated in KU
// independent chains.
template <int NC>
struct XSlice {
    float4 lo[NC], hi[NC];
};

// x chunks (8 elements) of this lane for KU units: chunk u * 64 + lane (bf16
// units), chunks 2 (u * 64 + lane) and 2 (u * 64 + lane) + 1 (FP8 units)
template <int KU, bool FP8>
__device__ __forceinline__ void load_xslice(const Ctx& cx, const LDS float* xb, int xstride,
                                            XSlice<FP8 ? 2 * KU : KU>& x) {
    if constexpr (FP8) {
#pragma unroll
        for (int c = 0; c < 2 * KU; ++c) {
            const int q = 2 * ((c >> 1) * 64 + cx.lane) + (c & 1);
            x.lo[c] = lds_f4(xb + 4 * q);
            x.hi[c] = lds_f4(xb + 4 * ((xstride >> 3) + q));
        }
    } else {
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            x.lo[u] = lds_f4(xb + 4 * (u * 64 + cx.lane));
            x.hi[u] = lds_f4(xb + 4 * ((xstride >> 3) + u * 64 + cx.lane));
        }
    }
}

template <int KU, int NROWS, bool FP8>
__device__ __forceinline__ void rowgroup_dot_b1(Ctx& cx, const Lds& s, Stream& st,
                                                const XSlice<FP8 ? 2 * KU : KU>& x, uint32_t ru, RowOut& out) {
#pragma unroll
    for (int r = 0; r < NROWS; ++r) {
        ring_wait(cx, s, st, st.unit + KU);
        uint4 w[KU];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            uint32_t sl = st.slot + u;
            sl = sl >= ru ? sl - ru : sl;
            w[u] = lds_u4(s.ring + ((size_t)cx.wave * ru + sl) * UNIT_BYTES + cx.lane * 16);
        }
        float acc[KU];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            if constexpr (FP8) acc[u] = dot16_fp8(w[u], x.lo[2 * u], x.hi[2 * u], x.lo[2 * u + 1], x.hi[2 * u + 1]);
            else acc[u] = dot8(w[u], x.lo[u], x.hi[u]);
        }
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
// for each of the NB batch rows (x read from LDS); the path for batch sizes
// above one.  NB is a template parameter so that a unit's 2 NB x loads are
// issued together and its NB product chains interleave.
// x of one unit for batch row b: (lo, hi) of chunk u * 64 + lane (bf16), and
// for FP8 units also (lo2, hi2) of the next chunk
template <bool FP8>
__device__ __forceinline__ float unit_dot(const uint4 w, const LDS float* xl, int xs, int b) {
    const LDS float* xr = xl + b * xs;
    if constexpr (FP8)
        return dot16_fp8(w, lds_f4(xr), lds_f4(xr + (xs >> 1)), lds_f4(xr + 4), lds_f4(xr + (xs >> 1) + 4));
    else
        return dot8(w, lds_f4(xr), lds_f4(xr + (xs >> 1)));
}

template <int NROWS, int NB, bool FP8>
__device__ __forceinline__ void rowgroup_dot(Ctx& cx, const Lds& s, Stream& st, const LDS float* xb, int ku,
                                             RowOut& out) {
    const int xs = (int)uni((uint32_t)cx.p->xstride);
    if constexpr (NROWS == 2) {  // the rows' units alternate in the stream: one x read serves both
        float a0[NB], a1[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) a0[b] = a1[b] = 0.f;
        for (int u = 0; u < ku; ++u) {
            const uint4 w0 = ring_take(cx, s, st);
            ring_advance(cx, st);
            const uint4 w1 = ring_take(cx, s, st);
            ring_advance(cx, st);
            const LDS float* xl = xb + 4 * (FP8 ? 2 * (u * 64 + cx.lane) : u * 64 + cx.lane);
            if constexpr (FP8) {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const LDS float* xr = xl + b * xs;
                    const float4 l0 = lds_f4(xr), h0 = lds_f4(xr + (xs >> 1)), l1 = lds_f4(xr + 4),
                                 h1 = lds_f4(xr + (xs >> 1) + 4);
                    a0[b] += dot16_fp8(w0, l0, h0, l1, h1);
                    a1[b] += dot16_fp8(w1, l0, h0, l1, h1);
                    CBAR();  // one batch row's x live at a time (register budget)
                }
            } else {
                float4 lo[NB], hi[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    lo[b] = lds_f4(xl + b * xs);
                    hi[b] = lds_f4(xl + b * xs + (xs >> 1));
                }
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    a0[b] += dot8(w0, lo[b], hi[b]);
                    a1[b] += dot8(w1, lo[b], hi[b]);
                }
            }
            if ((u & 1) == 1 || u == ku - 1) ring_release(cx, s, st);
        }
        float m0 = 0.f, m1 = 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float t0 = wave_sum(a0[b]), t1 = wave_sum(a1[b]);
            m0 = cx.lane == b ? t0 : m0;
            m1 = cx.lane == b ? t1 : m1;
        }
        out.mine[0] = m0;
        out.mine[1] = m1;
        return;
    }
#pragma unroll
    for (int r = 0; r < NROWS; ++r) {
        float acc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = 0.f;
        for (int u = 0; u < ku; ++u) {
            const uint4 w = ring_take(cx, s, st);
            const LDS float* xl = xb + 4 * (FP8 ? 2 * (u * 64 + cx.lane) : u * 64 + cx.lane);
            if constexpr (FP8) {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    acc[b] += unit_dot<true>(w, xl, xs, b);
                    CBAR();  // one batch row's x live at a time (register budget)
                }
            } else {
                float4 lo[NB], hi[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    lo[b] = lds_f4(xl + b * xs);
                    hi[b] = lds_f4(xl + b * xs + (xs >> 1));
                }
#pragma unroll
                for (int b = 0; b < NB; ++b) acc[b] += dot8(w, lo[b], hi[b]);
            }
            ring_advance(cx, st);
            if ((u & 3) == 3 || u == ku - 1) ring_release(cx, s, st);
        }
        float mine = 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float t = wave_sum(acc[b]);
            mine = cx.lane == b ? t : mine;
        }
        out.mine[r] = mine;
    }
}

template <int NROWS, bool FP8>
__device__ __forceinline__ void rowgroup_dot_batch(Ctx& cx, const Lds& s, Stream& st, const LDS float* xb, int ku,
                                                   RowOut& out) {
    if constexpr (!TU_BATCHED) {  // the batch-1 build: one batch row (heads whose rows are not
        // 2 or 4 units long take this general path at batch 1)
        rowgroup_dot<NROWS, 1, FP8>(cx, s, st, xb, ku, out);
        return;
    }
    if constexpr (FP8) {  // FP8 handles take at most four batch rows (register budget)
        switch (cx.p->B) {
        case 1: rowgroup_dot<NROWS, 1, true>(cx, s, st, xb, ku, out); break;
        case 2: rowgroup_dot<NROWS, 2, true>(cx, s, st, xb, ku, out); break;
        case 3: rowgroup_dot<NROWS, 3, true>(cx, s, st, xb, ku, out); break;
        default: rowgroup_dot<NROWS, 4, true>(cx, s, st, xb, ku, out); break;
        }
        return;
    }
    switch (cx.p->B) {
    case 1: rowgroup_dot<NROWS, 1, FP8>(cx, s, st, xb, ku, out); break;
    case 2: rowgroup_dot<NROWS, 2, FP8>(cx, s, st, xb, ku, out); break;
    case 3: rowgroup_dot<NROWS, 3, FP8>(cx, s, st, xb, ku, out); break;
    case 4: rowgroup_dot<NROWS, 4, FP8>(cx, s, st, xb, ku, out); break;
    case 5: rowgroup_dot<NROWS, 5, FP8>(cx, s, st, xb, ku, out); break;
    case 6: rowgroup_dot<NROWS, 6, FP8>(cx, s, st, xb, ku, out); break;
    case 7: rowgroup_dot<NROWS, 7, FP8>(cx, s, st, xb, ku, out); break;
    default: rowgroup_dot<NROWS, 8, FP8>(cx, s, st, xb, ku, out); break;
    }
}

struct Step {  // per-launch batch inputs, lane b holds row b
    int tok, pos;
    const int32_t* tokens;
    const int32_t* positions;
    uint16_t* kv;
    float* logits;
};

// ------------------------------------------------------------ gather wave --
//
// The gather wave stages every instruction's cross-CU inputs in one of nslot
// (1 to 3) LDS buffer sets, up to nslot - 1 instructions ahead of the compute
// waves (the sets rotate by instruction), so the compute waves start each instruction
// with a single LDS counter check instead of polling remote memory and
// meeting at a barrier.  For RMSNorm inputs it also sums the squares of the
// raw rows and stores x * gain.

// Reads the n (even) tagged words at base, two adjacent words per lane per
// 16-byte load and 128 * NB words per round, polling until every tag carries
// this step's epoch; put(k, v_k, v_k+1, gain pair) stores them.  With GAIN,
// the bf16 gain pair at gain + k is loaded alongside.  Buffer loads keep the
// addresses in scalar registers; their range check returns zeros past n.
constexpr uint32_t RSRC_WORD3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9)
constexpr int CPOL_SC1 = 16;                 // device-coherent load: bypasses the non-coherent L2 copy

template <int NB, bool GAIN, class Put>
__device__ __forceinline__ void gather_region(Ctx& cx, const uint64_t* base, int n, const uint16_t* gain, Put&& put) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, n * 8, RSRC_WORD3);
    __amdgpu_buffer_rsrc_t rg = rs;
    if (GAIN) rg = __builtin_amdgcn_make_buffer_rsrc((void*)gain, (short)0, n * 2, RSRC_WORD3);
    const uint32_t ep = cx.epoch;
    for (int k0 = 0; k0 < n; k0 += 128 * NB) {
        u32x4 w[NB];
        uint32_t g[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int k = k0 + j * 128 + 2 * cx.lane;
            w[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, k * 8, 0, CPOL_SC1);
            if (GAIN) g[j] = __builtin_amdgcn_raw_buffer_load_b32(rg, k * 2, 0, 0);
        }
        uint32_t spins = 0;
        while (true) {
            bool stale = false;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int k = k0 + j * 128 + 2 * cx.lane;
                stale |= k < n && (w[j].y != ep || w[j].w != ep);
            }
            if (!any_lane(stale)) break;
            if (!keep_waiting(cx, spins, 0x50000000u | (uint32_t)k0)) return;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int k = k0 + j * 128 + 2 * cx.lane;
                if (k < n && (w[j].y != ep || w[j].w != ep))
                    w[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, k * 8, 0, CPOL_SC1);
            }
        }
        if (cx.trace) cx.t_acq = rtime();  // every tag current
        // put(kb, ...) stores pair k = kb + 2 * lane, kb = k0 + 128 j; a full
        // round needs no per-pair bounds test
        if (k0 + 128 * NB <= n) {
#pragma unroll
            for (int j = 0; j < NB; ++j)
                put(k0 + j * 128, __uint_as_float(w[j].x), __uint_as_float(w[j].z), GAIN ? g[j] : 0x3f803f80u);
        } else {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int k = k0 + j * 128 + 2 * cx.lane;
                if (k < n) put(k0 + j * 128, __uint_as_float(w[j].x), __uint_as_float(w[j].z), GAIN ? g[j] : 0x3f803f80u);
            }
        }
    }
}

constexpr int GATHER_NB = 16;      // 16-byte loads per lane per polling round (2048 words)
constexpr int GATHER_NB_ATTN = 6;  // (G + 2) * D <= 768 words
#ifndef GATHER_NB_COMPUTE
#define GATHER_NB_COMPUTE 8          // compute waves staging their own x row (1024 words a round)
#endif

// x[b][k] = raw[k] * gain[k] for one batch row b in the x-buffer layout, plus zero padding up
// to kpad; ss_out[b] = sum_k raw[k]^2 when ss_out is given.
template <int NB, bool GAIN>
__device__ __forceinline__ void gather_x_row(Ctx& cx, int b, int K, int kpad, const uint64_t* raw,
                                             const uint16_t* gain, LDS float* xb, LDS float* ss_out) {
    const int xs = (int)uni((uint32_t)cx.p->xstride);
    float ss = 0.f;
    // lane l stores pairs k = k0 + 2l (k0 a multiple of 128): one base address per lane
    LDS float* xl = xb + xidx(xs, b, 2 * cx.lane);
    gather_region<NB, GAIN>(cx, raw, K, gain, [&](int kb, float v0, float v1, uint32_t gp) {
        ss = fmaf(v0, v0, ss);
        ss = fmaf(v1, v1, ss);
        LDS float* x = xl + (kb >> 1);  // k, k+1 adjacent
        x[0] = v0 * bf_lo(gp);
        x[1] = v1 * bf_hi(gp);
    });
    for (int k = K + cx.lane; k < kpad; k += 64) xb[xidx(xs, b, k)] = 0.f;
    if (ss_out) {
        ss = wave_sum(ss);
        if (cx.lane == 0) ss_out[b] = ss;
    }
}

// Embedding rows (bf16, written before the launch: no tags) as the input of
// the first layer's RMSNorm.
__device__ __forceinline__ void gather_embed(Ctx& cx, const Step& sp, int kpad, const uint16_t* gain, LDS float* xb,
                                             LDS float* ss_out) {
    CParams& p = *cx.p;
    const int H = p.H, xs = (int)uni((uint32_t)p.xstride);
    for (int b = 0; b < p.B; ++b) {
        const int tok = __builtin_amdgcn_readlane(sp.tok, b);
        const uint32_t* row = (const uint32_t*)(p.embed + (size_t)tok * H);  // H even: bf16 pairs
        float ss = 0.f;
        for (int k0 = 0; k0 < H; k0 += 128 * GATHER_NB) {
            uint32_t e[GATHER_NB], g[GATHER_NB];
#pragma unroll
            for (int j = 0; j < GATHER_NB; ++j) {
                const int k = k0 + j * 128 + 2 * cx.lane;
                e[j] = k < H ? gld(row + k / 2) : 0u;
                g[j] = k < H ? gld((const uint32_t*)(gain + k)) : 0u;
            }
#pragma unroll
            for (int j = 0; j < GATHER_NB; ++j) {
                const int k = k0 + j * 128 + 2 * cx.lane;
                if (k < H) {
                    const float v0 = bf_lo(e[j]), v1 = bf_hi(e[j]);
                    ss = fmaf(v0, v0, ss);
                    ss = fmaf(v1, v1, ss);
                    LDS float* x = xb + xidx(xs, b, k);
                    x[0] = v0 * bf_lo(g[j]);
                    x[1] = v1 * bf_hi(g[j]);
                }
            }
        }
        for (int k = H + cx.lane; k < kpad; k += 64) xb[xidx(xs, b, k)] = 0.f;
        ss = wave_sum(ss);
        if (cx.lane == 0) ss_out[b] = ss;
    }
}

// n tagged words at src (any alignment) into dst[0 .. n), 4 per lane per round.
__device__ __forceinline__ void gather_words(Ctx& cx, const uint64_t* src, int n, LDS float* dst) {
    for (int i0 = 0; i0 < n; i0 += 256) {
        uint64_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = i0 + j * 64 + cx.lane;
            w[j] = i < n ? ld_tag(src + i) : ((uint64_t)cx.epoch << 32);
        }
        uint32_t spins = 0;
        while (true) {
            bool stale = false;
#pragma unroll
            for (int j = 0; j < 4; ++j) stale |= tag_of(w[j]) != cx.epoch;
            if (!any_lane(stale)) break;
            if (!keep_waiting(cx, spins, 0x58000000u | (uint32_t)i0)) return;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (tag_of(w[j]) != cx.epoch) w[j] = ld_tag(src + i0 + j * 64 + cx.lane);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = i0 + j * 64 + cx.lane;
            if (i < n) dst[i] = val_of(w[j]);
        }
    }
}

// Epilogue inputs staged next to x (when side buffers are enabled):
//   QKV: side[b * D + 2 i + {0, 1}] = (cos, sin) of pair i at position pos_b
//   O:   side[b * nrg + j] = residual stream entering the layer, row rg0 + j
//   last down chunk: side[b * nrg + j] = residual after attention, row rg0 + j
__device__ __forceinline__ void gather_side(Ctx& cx, const Step& sp, const Inst& in, LDS float* sd) {
    CParams& p = *cx.p;
    const int B = p.B, H = p.H, l = in.layer, nrg = (int)in.nrg, rg0 = (int)in.rg0;
    if (in.op == OP_RMS_QKV_ROPE) {
        return;  // the step's RoPE rows were loaded at launch
    } else if (in.op == OP_O_PROJ_RES) {
        if (cx.resident && l > 0) return;  // the residual rows are the CU's own, kept in LDS
        for (int b = 0; b < B; ++b) {
            if (l == 0) {
                const uint16_t* e = p.embed + (size_t)__builtin_amdgcn_readlane(sp.tok, b) * H + rg0;
                for (int j = cx.lane; j < nrg; j += 64) sd[b * nrg + j] = bf2f(gld(e + j));
            } else {
                gather_words(cx, p.hout + ((size_t)(l - 1) * B + b) * H + rg0, nrg, sd + b * nrg);
            }
        }
    } else if (in.op == OP_DOWN_RES && in.a == p.n_chunk - 1 && !cx.resident) {
        for (int b = 0; b < B; ++b) gather_words(cx, p.hmid + ((size_t)l * B + b) * H + rg0, nrg, sd + b * nrg);
    }
}


// Stages the inputs of one instruction in xb (see the op bodies for layouts).
// (FP8 weights: units of 1024 elements, so the zero padding of x covers those)
// With several batch rows the compute waves stage the x rows of the GEMV inputs themselves, wave
// w row w, so the rows' polls run at once instead of one after another on the gather wave (one
// round trip per instruction instead of B); the gather wave still frees the buffer set, stages
// the side inputs and raises the ready flag.  The first layer's QKV input (embedding rows, no
// tags) stays with the gather wave.
__device__ __forceinline__ bool rows_by_compute(CParams& p, const Inst& in) {
    if (!TU_BATCHED || p.B == 1) return false;
    switch (in.op) {
    case OP_RMS_QKV_ROPE: return in.layer > 0;
    case OP_RMS_LM_HEAD:
    case OP_RMS_UP_GATE:
    case OP_O_PROJ_RES:
    case OP_DOWN_RES: return true;
    default: return false;
    }
}

template <bool FP8>
__device__ __forceinline__ void gather_inst(Ctx& cx, const Step& sp, const Inst& in, LDS float* xb, LDS float* ss) {
    constexpr int NB = GATHER_NB;
    const int b0 = 0, bstep = 1;
    constexpr int EPU = FP8 ? FP8_UNIT_ELEMS : UNIT_ELEMS;
    CParams& p = *cx.p;
    const int B = p.B, H = p.H, l = in.layer;
    switch (in.op) {
    case OP_RMS_QKV_ROPE:
    case OP_RMS_LM_HEAD: {
        const int src_layer = in.op == OP_RMS_LM_HEAD ? p.L : l;  // residual stream entering this layer
        const uint16_t* gain = in.op == OP_RMS_LM_HEAD ? p.gain_final : p.gain_attn + (size_t)l * H;
        const int kpad = p.ku_h * EPU;
        if (src_layer == 0) {
            gather_embed(cx, sp, kpad, gain, xb, ss);
        } else {
            const uint64_t* src = p.hout + (size_t)(src_layer - 1) * B * H;
            for (int b = b0; b < B; b += bstep) gather_x_row<NB, true>(cx, b, H, kpad, src + (size_t)b * H, gain, xb, ss);
        }
        break;
    }
    case OP_RMS_UP_GATE: {
        const uint64_t* src = p.hmid + (size_t)l * B * H;
        for (int b = b0; b < B; b += bstep)
            gather_x_row<NB, true>(cx, b, H, p.ku_h * EPU, src + (size_t)b * H, p.gain_mlp + (size_t)l * H, xb, ss);
        break;
    }
    case OP_O_PROJ_RES: {
        const int K = p.Hq * p.D;
        const uint64_t* src = p.attn + (size_t)l * B * K;
        for (int b = b0; b < B; b += bstep)
            gather_x_row<NB, false>(cx, b, K, p.ku_q * EPU, src + (size_t)b * K, nullptr, xb, nullptr);
        break;
    }
    case OP_DOWN_RES: {
        const int c0 = p.chunk_begin[in.a], K = p.chunk_begin[in.a + 1] - c0;
        const uint64_t* src = p.act + (size_t)l * B * p.F + c0;
        for (int b = b0; b < B; b += bstep)
            gather_x_row<NB, false>(cx, b, K, p.ku_f * EPU, src + (size_t)b * p.F, nullptr, xb, nullptr);
        break;
    }
    case OP_ATTENTION: {
        // qs [G][D] (pre-scaled by 1/sqrt(D)), kn [D], vn [D]: one contiguous block
        const int b = in.a, g = in.b, D = p.D, nq = p.G * D;
        const uint64_t* src = p.qkv + (((size_t)l * B + b) * p.Hkv + g) * (size_t)(p.G + 2) * D;
        const float sc = p.inv_sqrt_d;
        gather_region<GATHER_NB_ATTN, false>(cx, src, nq + 2 * D, nullptr, [&](int kb, float v0, float v1, uint32_t) {
            const int i = kb + 2 * cx.lane;
            const float f = i < nq ? sc : 1.f;  // nq even: a pair never straddles q and k
            xb[i] = v0 * f;
            xb[i + 1] = v1 * f;
        });
        break;
    }
    default: {  // OP_ATTN_REDUCE: the n_split partials (m, l, o[D]) of (row, head)
        const int b = in.a, head = in.b, W = p.D + 2;
        const uint64_t* src = p.part + (((size_t)l * B + b) * p.Hq + head) * p.n_split * W;
        gather_region<GATHER_NB, false>(cx, src, p.n_split * W, nullptr, [&](int kb, float v0, float v1, uint32_t) {
                                           const int i = kb + 2 * cx.lane;
                                           xb[i] = v0;
                                           xb[i + 1] = v1;
                                       });
        break;
    }
    }
}

// Compute wave side of rows_by_compute: this wave stages x row b = cx.wave (if b < B) of a GEMV
// instruction's input (only the GEMV cases, with fewer loads per round than the gather wave).
template <bool FP8>
__device__ __forceinline__ void gather_own_row(Ctx& cx, const Inst& in, LDS float* xb, LDS float* ss) {
    constexpr int EPU = FP8 ? FP8_UNIT_ELEMS : UNIT_ELEMS;
    constexpr int NB = GATHER_NB_COMPUTE;
    CParams& p = *cx.p;
    const int B = p.B, H = p.H, l = in.layer, b = cx.wave;
    if (b >= B) return;
    const uint64_t* raw;
    const uint16_t* gain = nullptr;
    int K, kpad;
    if (in.op == OP_RMS_QKV_ROPE || in.op == OP_RMS_LM_HEAD || in.op == OP_RMS_UP_GATE) {
        const bool up = in.op == OP_RMS_UP_GATE;
        const int src_layer = in.op == OP_RMS_LM_HEAD ? p.L : l;  // (> 0: the embedding rows stay with the gather wave)
        raw = up ? p.hmid + ((size_t)l * B + b) * H : p.hout + ((size_t)(src_layer - 1) * B + b) * H;
        gain = up ? p.gain_mlp + (size_t)l * H : in.op == OP_RMS_LM_HEAD ? p.gain_final : p.gain_attn + (size_t)l * H;
        K = H;
        kpad = p.ku_h * EPU;
        gather_x_row<NB, true>(cx, b, K, kpad, raw, gain, xb, ss);
    } else if (in.op == OP_O_PROJ_RES) {
        K = p.Hq * p.D;
        gather_x_row<NB, false>(cx, b, K, p.ku_q * EPU, p.attn + ((size_t)l * B + b) * K, nullptr, xb, nullptr);
    } else {  // OP_DOWN_RES
        const int c0 = p.chunk_begin[in.a];
        K = p.chunk_begin[in.a + 1] - c0;
        gather_x_row<NB, false>(cx, b, K, p.ku_f * EPU, p.act + ((size_t)l * B + b) * p.F + c0, nullptr, xb, nullptr);
    }
}

// Consecutive instructions of one CU that read the same full input vector
// (the up/gate chunks of a layer, several row tiles of one GEMV op) share it:
// the gather wave copies it from the buffer set it staged last instead of
// polling it from global memory again (one round trip saved per instruction).
__device__ __forceinline__ uint32_t input_key(const Inst& in) {
    const bool whole = in.op == OP_RMS_QKV_ROPE || in.op == OP_RMS_UP_GATE || in.op == OP_RMS_LM_HEAD ||
                       in.op == OP_O_PROJ_RES;
    return whole ? (uint32_t)in.op | ((uint32_t)in.layer << 8) : 0u;
}

__device__ __forceinline__ void copy_staged(const Ctx& cx, const LDS float* from, LDS float* to, int n,
                                            const LDS float* ss_from, LDS float* ss_to, int B) {
    for (int i = cx.lane * 4; i < n; i += 64 * 4) *(LDS f32x4*)(to + i) = *(const LDS f32x4*)(from + i);
    if (cx.lane < B) ss_to[cx.lane] = ss_from[cx.lane];
}

__device__ __forceinline__ Inst decode_inst(const u32x4 raw) {
    Inst in;
    in.op = (uint16_t)(raw.x & 0xffffu);
    in.layer = (uint16_t)(raw.x >> 16);
    in.rg0 = raw.y;
    in.nrg = raw.z;
    in.a = (uint16_t)(raw.w & 0xffffu);
    in.b = (uint16_t)(raw.w >> 16);
    return in;
}

// Gather wave g's loop over instructions pc0 + g, pc0 + g + NGATHER, ... of
// this CU's queue: the gather waves take turns, so one wave's poll round trip
// overlaps another's staging.
template <bool FP8>
__device__ __forceinline__ void gatherer(Ctx& cx, const Lds& s, const Step& sp, uint32_t qb, uint32_t pc0,
                                         uint32_t pc1, int g) {
    CParams& p = *cx.p;
    __builtin_amdgcn_s_setprio(MK_LOADER_PRIO);
    const CONST_AS u32x4* iq = (const CONST_AS u32x4*)(p.insts + uni(qb));
    const uint32_t nslot = uni((uint32_t)p.nslot);
    uint32_t slot = (uint32_t)g % nslot;
    uint32_t prev_key = 0, prev_slot = 0;  // input of the instruction this wave staged last
    {
        // the (cos, sin) rows of the step's positions, for every QKV epilogue of the launch (read
        // after the ready flag of a QKV instruction, which this wave publishes later)
        const int D = p.D;
        for (int b = 0; b < p.B; ++b) {
            const float* rope = p.rope + (size_t)__builtin_amdgcn_readlane(sp.pos, b) * D;
            for (int i = cx.lane; i < D; i += 64) s.rope[b * D + i] = gld(rope + i);
        }
        vm_drain();
    }
    for (uint32_t pc = pc0 + g; pc < pc1; pc += NGATHER, slot = (slot + NGATHER) % nslot) {
        const uint32_t r = pc - pc0;
        const u32x4 raw = iq[pc];
        if (r >= nslot) {  // buffer set `slot` held instruction r - nslot: wait until every compute wave is done with it
            // (one counter per wave: a wave with less work in an instruction may
            // run ahead, so a shared count could reach the total too early)
            const uint32_t need = r - nslot + 1;
            uint32_t spins = 0;
            while (any_lane(cx.lane < NW && lds_ld(s.done + (cx.lane < NW ? cx.lane : 0)) < need))
                if (!keep_waiting<2>(cx, spins, 0x60000000u | r)) break;
        }
        if (uni(cx.aborted)) break;
        const Inst in = decode_inst(raw);
        cx.pc = pc;
        cx.op = in.op;
        const uint64_t t0 = cx.trace ? rtime() : 0;
        cx.t_acq = t0;
        // side inputs first: each was complete before the main input's producers
        // began, so their round trip never waits behind the main poll
        if (p.side_floats) gather_side(cx, sp, in, sslot(s, p, slot));
        const bool by_compute = rows_by_compute(p, in);
        const uint32_t key = by_compute ? 0u : input_key(in);
        if (by_compute) {
            // the compute waves stage the x rows
        } else if (NGATHER == 1 && key != 0 && key == prev_key) {  // its buffer set still holds it:
            // the wave refills a set only nslot instructions later, after this copy (with one set,
            // the data is already in place)
            if (slot != prev_slot)
                copy_staged(cx, xslot(s, p, prev_slot), xslot(s, p, slot), p.B * (int)uni((uint32_t)p.xstride),
                            s.ss + prev_slot * MAX_BATCH, s.ss + slot * MAX_BATCH, p.B);
        } else {
            gather_inst<FP8>(cx, sp, in, xslot(s, p, slot), s.ss + slot * MAX_BATCH);
        }
        prev_key = key;
        prev_slot = slot;
        if (uni(cx.aborted)) break;
        CBAR();
        if (cx.lane == 0) lds_st(s.ready + slot, r + 1);  // after the staged data (LDS requests of a wave stay ordered)
        if (cx.trace && cx.lane == 0) {
            GLB uint64_t* rec = (GLB uint64_t*)p.trace + (size_t)(qb + pc) * TRACE_SLOTS + 1 + TRACE_WAVE_SLOTS * NW;
            rec[0] = t0;
            rec[1] = cx.t_acq;
            rec[2] = rtime();
        }
    }
}

// Compute-wave side: wait until instruction r's inputs are staged (in buffer set cx.slot).
__device__ __forceinline__ void wait_inputs(Ctx& cx, const Lds& s, uint32_t r) {
    const uint64_t t0 = cx.prof ? cycles() : 0;
    uint32_t spins = 0;
#ifndef MK_INPUT_SLEEP
#define MK_INPUT_SLEEP MK_SLEEP
#endif
    while (uni(lds_ld(s.ready + cx.slot)) != r + 1)
        if (!keep_waiting<MK_INPUT_SLEEP>(cx, spins, 0x70000000u | r)) break;
    CBAR();
    if (cx.prof) cx.cnt[2] += cycles() - t0;
    mark_acquired(cx);
    mark_inputs(cx);
}

// ------------------------------------------------------------ GEMV ops ------

// Down-projection partial sums of a wave's first DREG row-groups stay in
// registers across the chunk instructions of a layer (lane b: batch row b);
// further row-groups use the global accumulator.
constexpr int DREG = 4;
struct DownAcc {
    float r[DREG];
};

// Up/gate instructions: one per CU and layer, its share of every down-projection chunk, chunk
// after chunk.  CU slot t's share of chunk c is rows [r0, r0 + n) (the schedule builder splits
// the same way); values below 2^24, so the products stay in 32 bits.
__device__ __forceinline__ uint32_t ug_share(CParams& p, uint32_t t, int c, uint32_t& r0) {
    const uint32_t c0 = (uint32_t)p.chunk_begin[c], len = (uint32_t)p.chunk_begin[c + 1] - c0;
    const uint32_t ncu = (uint32_t)p.ncu;
    r0 = c0 + len * t / ncu;
    return c0 + len * (t + 1) / ncu - r0;
}

// KU > 0: batch-1 path with KU units per row (x slice in registers);
// KU == 0: general path.
template <int KU, bool FP8, bool GREEDY, bool ABLATE>
__device__ __forceinline__ void op_gemv(Ctx& cx, const Lds& s, Stream& st, uint32_t r, uint32_t slot, const Inst& in,
                                        LDS float* xb, const Step& sp, DownAcc& da, uint32_t& seq) {
    CParams& p = *cx.p;
    const int B = p.B, H = p.H, l = in.layer;
    const int ku = in.op == OP_O_PROJ_RES ? p.ku_q : in.op == OP_DOWN_RES ? p.ku_f : p.ku_h;
    const uint32_t row_end = st.unit + in.b;  // the instruction's unit-rows end here in every ring
    // FP8 weights: each row sum times its row's scale; lane j holds the pair of row-group
    // cx.wave + (j0 + j) * NW, loaded once per 64 row-groups of the wave before the inputs are
    // awaited, and row-group ri's pair is read out with readlane
    float2 rsc = make_float2(1.f, 1.f);
    const float* rgs = nullptr;
    auto load_rsc = [&](uint32_t j0) {
        const uint32_t i = cx.wave + (j0 + cx.lane) * NW;
        uint32_t row = i;
        if (in.op == OP_RMS_UP_GATE) {  // the table is indexed by row: find row-group i's
            uint32_t base = 0;
            for (int c = 0; c < p.n_chunk; ++c) {
                uint32_t r0;
                const uint32_t n = ug_share(p, in.rg0, c, r0);
                if (i >= base && i < base + n) row = r0 + (i - base);
                base += n;
            }
        }
        rsc = i < in.nrg ? *(const float2*)(rgs + 2 * (size_t)row) : make_float2(1.f, 1.f);
    };
    if constexpr (FP8) {
        const int k = in.op == OP_RMS_QKV_ROPE ? 0 : in.op == OP_O_PROJ_RES ? 1 : in.op == OP_RMS_UP_GATE ? 2 : 3;
        const size_t base = in.op == OP_RMS_LM_HEAD ? (size_t)p.L * p.rgs_stride
                                                    : (size_t)l * p.rgs_stride + p.rgs_off[k];
        rgs = p.rgscale + 2 * (base + (in.op == OP_RMS_UP_GATE ? 0u : in.rg0));
        load_rsc(0);
    }
    // x = raw input * gain, staged by the gather wave (with several batch rows: by the compute
    // waves, one row each, once the gather wave has handed over the buffer set); lane b: RMSNorm
    // scale of batch row b
    wait_inputs(cx, s, r);
    if (cx.aborted) return;
    if (rows_by_compute(p, in)) {
        gather_own_row<FP8>(cx, in, xb, s.ss + slot * MAX_BATCH);
        cbar(cx, s, seq);
        if (cx.aborted) return;
    }
    float scale = 1.f;
    if ((in.op == OP_RMS_QKV_ROPE || in.op == OP_RMS_LM_HEAD || in.op == OP_RMS_UP_GATE) && cx.lane < B)
        scale = rsqrtf(s.ss[slot * MAX_BATCH + cx.lane] * (1.0f / (float)H) + p.eps);

    XSlice<KU == 0 ? 1 : (FP8 ? 2 * KU : KU)> xs;
    const uint32_t ru = __builtin_amdgcn_readfirstlane((uint32_t)p.ring_units);
    if constexpr (KU > 0) load_xslice<KU, FP8>(cx, xb, __builtin_amdgcn_readfirstlane(p.xstride), xs);
    // ablation build, this opcode switched off: the row sums are 0 (units passed over unread)
    const bool off = ABLATE && in.op == p.ablate_op;
    auto dot1 = [&](RowOut& o) {
        if (ABLATE && off) {
            ring_skip(cx, s, st, (uint32_t)ku);
            o.mine[0] = o.mine[1] = 0.f;
            return;
        }
        if constexpr (KU > 0) rowgroup_dot_b1<KU, 1, FP8>(cx, s, st, xs, ru, o);
        else rowgroup_dot_batch<1, FP8>(cx, s, st, xb, ku, o);
    };
    auto dot2 = [&](RowOut& o) {
        if (ABLATE && off) {
            ring_skip(cx, s, st, 2u * (uint32_t)ku);
            o.mine[0] = o.mine[1] = 0.f;
            return;
        }
        if constexpr (KU > 0) rowgroup_dot_b1<KU, 2, FP8>(cx, s, st, xs, ru, o);
        else rowgroup_dot_batch<2, FP8>(cx, s, st, xb, ku, o);
    };
    float2 sc = make_float2(1.f, 1.f);
    auto fp8_scale = [&](RowOut& o) {
        o.mine[0] *= sc.x;
        o.mine[1] *= sc.y;
    };

    // ---- this wave's row-groups; lane b < B finishes batch row b
    const int D = p.D, half = D / 2;
    const bool lane_row = cx.lane < B;
    const int b = lane_row ? cx.lane : 0;
    const int nrg = (int)in.nrg;
    const LDS float* sd = p.side_floats ? sslot(s, p, slot) : nullptr;  // staged epilogue inputs
    // up/gate: chunk ug_c of the current row-group, whose rows [ug_r0, ug_r0 + ug_n) are the
    // instruction's row-groups [ug_base, ug_base + ug_n)
    uint32_t ug_c = 0, ug_base = 0, ug_r0 = 0, ug_n = 0;
    if (in.op == OP_RMS_UP_GATE) ug_n = ug_share(p, in.rg0, 0, ug_r0);
    for (uint32_t ri = 0;; ++ri) {
        const uint32_t i = cx.wave + ri * NW;
        if (i >= in.nrg) break;
        uint32_t rg = in.rg0 + i;
        if (in.op == OP_RMS_UP_GATE) {
            while (i >= ug_base + ug_n) {  // i < nrg: a later chunk holds it
                ug_base += ug_n;
                ug_n = ug_share(p, in.rg0, ++ug_c, ug_r0);
            }
            rg = ug_r0 + (i - ug_base);
        }
        if constexpr (FP8) {
            if (ri > 0 && (ri & 63) == 0) load_rsc(ri);
            sc.x = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rsc.x), (int)(ri & 63)));
            sc.y = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rsc.y), (int)(ri & 63)));
        }
        RowOut o;
        switch (in.op) {
        case OP_RMS_QKV_ROPE: {
            dot2(o);
            if constexpr (FP8) fp8_scale(o);
            if (lane_row) {
                const int pos = sp.pos;
                const float y1 = o.mine[0] * scale, y2 = o.mine[1] * scale;
                const int G = p.G, PG = (G + 2) * half;
                const int g = rg / PG, t = rg % PG;
                if (t < (G + 1) * half) {  // q or k: rotate the pair (ii, ii + D/2)
                    const int ii = t < G * half ? t % half : t - G * half;
                    const float2 cs = make_float2(s.rope[b * D + 2 * ii], s.rope[b * D + 2 * ii + 1]);
                    const float r1 = y1 * cs.x - y2 * cs.y, r2 = y2 * cs.x + y1 * cs.y;
                    uint64_t* blk = p.qkv + (((size_t)l * B + b) * p.Hkv + g) * (size_t)(G + 2) * D;
                    if (t < G * half) {
                        uint64_t* q = blk + (t / half) * D;
                        st_tag(q + ii, r1, cx.epoch);
                        st_tag(q + ii + half, r2, cx.epoch);
                    } else {
                        const uint16_t k1 = f2bf(r1), k2 = f2bf(r2);
                        uint16_t* kc = sp.kv + ((((size_t)l * 2 + 0) * B + b) * p.Hkv + g) * (size_t)p.max_seq * D + (size_t)pos * D;
                        gst(kc + ii, k1);
                        gst(kc + ii + half, k2);
                        uint64_t* kn = blk + G * D;
                        st_tag(kn + ii, bf2f(k1), cx.epoch);
                        st_tag(kn + ii + half, bf2f(k2), cx.epoch);
                    }
                } else {  // v: no rotation
                    const int ii = t - (G + 1) * half;
                    const uint16_t v1 = f2bf(y1), v2 = f2bf(y2);
                    uint16_t* vc = sp.kv + ((((size_t)l * 2 + 1) * B + b) * p.Hkv + g) * (size_t)p.max_seq * D + (size_t)pos * D;
                    gst(vc + ii, v1);
                    gst(vc + ii + half, v2);
                    uint64_t* vn = p.qkv + (((size_t)l * B + b) * p.Hkv + g) * (size_t)(G + 2) * D + (G + 1) * D;
                    st_tag(vn + ii, bf2f(v1), cx.epoch);
                    st_tag(vn + ii + half, bf2f(v2), cx.epoch);
                }
            }
            break;
        }
        case OP_O_PROJ_RES: {
            // residual stream entering layer l (complete before this layer's QKV began)
            float hin = 0.f;
            LDS float* res = s.res + (size_t)b * p.res_stride + i;  // this CU's row i (its own down-proj output)
            if (lane_row) {
                if (cx.resident && l > 0) hin = *res;
                else if (sd) hin = sd[b * nrg + i];
                else if (l == 0) hin = bf2f(gld_now(p.embed + (size_t)sp.tok * H + rg));
                else hin = wait_word(cx, p.hout + ((size_t)(l - 1) * B + b) * H + rg);
            }
            dot1(o);
            if constexpr (FP8) fp8_scale(o);
            if (lane_row) {
                const float hm = hin + o.mine[0];
                st_tag(p.hmid + ((size_t)l * B + b) * H + rg, hm, cx.epoch);
                if (cx.resident) *res = hm;  // read back by the last down-proj chunk of this layer
            }
            break;
        }
        case OP_RMS_UP_GATE: {
            dot2(o);
            if constexpr (FP8) fp8_scale(o);
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
            LDS float* res = s.res + (size_t)b * p.res_stride + i;  // this CU's row i (its own O-proj output)
            if (last && lane_row)
                hm = cx.resident ? *res : sd ? sd[b * nrg + i] : wait_word(cx, p.hmid + ((size_t)l * B + b) * H + rg);
            float* acc = p.dacc + (size_t)b * H + rg;  // global accumulator: this wave's lane b only
            float prev = 0.f;
            if (!first) {
                if (ri < DREG)
                    prev = ri == 0 ? da.r[0] : ri == 1 ? da.r[1] : ri == 2 ? da.r[2] : da.r[3];
                else if (lane_row)
                    prev = gld_now(acc);
            }
            dot1(o);
            if constexpr (FP8) fp8_scale(o);
            const float v = o.mine[0] + prev;
            if (last) {
                if (lane_row) {
                    st_tag(p.hout + ((size_t)l * B + b) * H + rg, hm + v, cx.epoch);
                    if (cx.resident) *res = hm + v;  // the residual entering the next layer's O-proj
                }
            } else if (ri < DREG) {
                if (ri == 0) da.r[0] = v;
                else if (ri == 1) da.r[1] = v;
                else if (ri == 2) da.r[2] = v;
                else da.r[3] = v;
            } else if (lane_row) {
                gst(acc, v);
            }
            break;
        }
        default: {  // OP_RMS_LM_HEAD (row-group rg: row rg, or rows 2 rg and 2 rg + 1 with lm_pairs)
            const int nr = TU_BATCHED && KU == 0 && p.lm_pairs ? 2 : 1;
            if (nr == 2) dot2(o);
            else dot1(o);
            if constexpr (FP8) fp8_scale(o);
            if (lane_row) {
                for (int k = 0; k < nr; ++k) {
                    const uint32_t row = nr == 2 ? 2 * rg + (uint32_t)k : rg;
                    const float v = o.mine[k] * scale;
                    gst(sp.logits + (size_t)b * p.V + row, v);
                    // the CU's best row so far (largest value, then lowest index); NaN is never selected
                    if constexpr (GREEDY)
                        if (v == v)
                            __hip_atomic_fetch_max(s.gkey + b, greedy_key(v, row), __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_WORKGROUP);
                }
            }
            break;
        }
        }
        if (cx.aborted) return;
    }
    // rows of this instruction that hold no units of this wave: skip them
    if (st.unit < row_end) {
        const uint32_t ru = uni((uint32_t)p.ring_units);
        st.slot = (st.slot + (row_end - st.unit)) % ru;
        st.unit = row_end;
        ring_release(cx, s, st);
    }
    mark_mid(cx);
}

// ------------------------------------------------------- attention ops ------

// One butterfly stage across lanes L and its partner L ^ stride: a lane whose stride bit is clear
// keeps the lower-destined value a plus its partner's a, the other keeps b plus the partner's
// b.  The exchanges are VALU lane permutations (gfx950's permlane swaps for strides 32 and 16,
// DPP within rows of 16 lanes below), not trips through the LDS crossbar.
template <int STRIDE>
__device__ __forceinline__ float bfly(float a, float b, int lane) {
    if constexpr (STRIDE == 32 || STRIDE == 16) {
        // swap(a, b) leaves lane L with (a of L, a of L + stride) when the bit is clear and
        // (b of L - stride, b of L) when it is set
        const auto r = STRIDE == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false)
                                    : __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
        const bool upper = (lane & STRIDE) != 0;
        const int x = __float_as_int(upper ? a : b);  // what the partner needs
        int y;
        if constexpr (STRIDE == 8) {
            y = __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false);  // row_ror:8 = lane ^ 8
        } else if constexpr (STRIDE == 4) {
            const int up = __builtin_amdgcn_update_dpp(0, x, 0x12C, 0xF, 0xF, false);  // from lane + 4
            const int dn = __builtin_amdgcn_update_dpp(0, x, 0x124, 0xF, 0xF, false);  // from lane - 4
            y = upper ? dn : up;
        } else if constexpr (STRIDE == 2) {
            y = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
        } else {
            y = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
        }
        return (upper ? b : a) + __int_as_float(y);
    }
}

// Split-KV partial attention of query heads g*G .. g*G+G-1 of batch row b over
// keys [j0, j1) of split s: writes (m, l, o[D]) with m the max score, l the
// sum of exp(score - m) and o the exp-weighted sum of V rows (unnormalised).
// Waves split the group's heads and 64-key blocks (the lane layouts within a
// block are described at the loads below).
template <int D, bool ABLATE>
__device__ __forceinline__ void op_attention_t(Ctx& cx, const Lds& s, uint32_t& seq, uint32_t r, const Inst& in,
                                               LDS float* xb,
                                               const Step& sp) {
    constexpr int NH = D / 64;       // 64-dim halves
    CParams& p = *cx.p;
    const int B = p.B, G = p.G, l = in.layer, b = in.a, g = in.b, split = (int)in.rg0;
    const int pos = __builtin_amdgcn_readlane(sp.pos, b);
    const int S = pos + 1;
    const int j0 = (int)((long long)split * S / p.n_split), j1 = (int)((long long)(split + 1) * S / p.n_split);
    LDS float* qs = xb;              // [G][D], pre-scaled by 1/sqrt(D)
    LDS float* kn = qs + G * D;      // [D] new K row (bf16 values)
    LDS float* vn = kn + D;          // [D] new V row
    LDS float* stt = vn + D;         // [NW][D + 2] per-wave (m, l, o), then [NW][64] weights
    const int gi = cx.wave % G, wph = NW / G, sub = cx.wave / G;
    const uint16_t* Kc = sp.kv + ((((size_t)l * 2 + 0) * B + b) * p.Hkv + g) * (size_t)p.max_seq * D;
    const uint16_t* Vc = sp.kv + ((((size_t)l * 2 + 1) * B + b) * p.Hkv + g) * (size_t)p.max_seq * D;
    const int nkeys = j1 - j0;

    // K and V rows written by earlier steps do not depend on this step: the first block's are
    // loaded before the wait for q.
    //
    // Lane layout in a block of 64 keys: load c (0..7) of a 64-dim half h has lane L read dims
    // 64h + 8(L%8) .. +7 of key 8c + L/8, so one load instruction covers eight whole 128-byte
    // lines.  A lane first holds eight partial scores (one per key it touched, over its dims);
    // a reduce-scatter over the eight lanes of its group leaves it with the whole score of key
    // 8(L%8) + L/8.  After the softmax the group's eight weights are shared through LDS, the
    // lane accumulates its eight keys into its dims, and a reduce-scatter over the eight
    // groups leaves it with output dims 64h + 8(L%8) + L/8.
    //
    // Registers hold two 64-key x 64-dim tiles.  64-dim heads keep a block's K and V in them
    // (one memory round trip per block: the next block's K is loaded once the scores are
    // taken, its V once the PV product is); 128-dim heads keep the two K halves, then the two
    // V halves (two round trips per block).
    //
    // The tiles are read with buffer loads whose range is the split's rows already in the cache,
    // [j0, min(j1, pos)): the hardware range check on the vector offset returns zeros for keys
    // past it (the row at pos, which comes from LDS, and the tail of the last block), so every
    // load of a tile shares one offset register.
    uint4 kr[8], vr[8];
    const int ch = cx.lane & 7, grp = cx.lane >> 3;
    const int ncached = min(j1, pos) - j0;  // keys of the split already in the cache
    const uint32_t nbytes = (uint32_t)ncached * (uint32_t)(D * 2);
    const __amdgpu_buffer_rsrc_t kres =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Kc + (size_t)j0 * D), (short)0, nbytes, RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t vres =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Vc + (size_t)j0 * D), (short)0, nbytes, RSRC_WORD3);
    auto load_blk = [&](uint4 (&r)[8], __amdgpu_buffer_rsrc_t rs, int kb, int h) {
        const uint32_t vo = (uint32_t)(((kb * 64 + grp) * D + h * 64 + ch * 8) * 2);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            // (a load whose eight keys are all past the range is not issued: the returns of a
            // wave's loads are in order, so it would only delay the ones after it)
            u32x4 w = {0, 0, 0, 0};
            if (kb * 64 + c * 8 < ncached) w = __builtin_amdgcn_raw_buffer_load_b128(rs, vo + (uint32_t)(c * 8 * D * 2), 0, 0);
            r[c] = make_uint4(w.x, w.y, w.z, w.w);
        }
    };
    // the new row's values are bf16 numbers held as fp32: their upper halves are the bf16 bits
    auto pack8 = [&](const LDS float* row) {
        const uint4 lo = lds_u4(row), hi = lds_u4(row + 4);
        return make_uint4((lo.x >> 16) | (lo.y & 0xffff0000u), (lo.z >> 16) | (lo.w & 0xffff0000u),
                          (hi.x >> 16) | (hi.y & 0xffff0000u), (hi.z >> 16) | (hi.w & 0xffff0000u));
    };
    // the row this step appended is not in the cache yet: its chunks come from LDS
    auto put_new = [&](uint4 (&r)[8], const LDS float* row, int rel) {
        const uint4 pk = pack8(row + ch * 8);
#pragma unroll
        for (int c = 0; c < 8; ++c)
            if (c * 8 + grp == rel) r[c] = pk;
    };
    if (sub * 64 < nkeys) {
        load_blk(kr, kres, sub, 0);
        if constexpr (NH == 1) load_blk(vr, vres, sub, 0);
        else load_blk(vr, kres, sub, 1);
    }

    // q of the group's heads (pre-scaled), then the new K and V rows, staged by the gather wave
    wait_inputs(cx, s, r);
    if (cx.aborted) return;
    if (ABLATE && p.ablate_op == OP_ATTENTION) {  // switched off: the partial of an all-zero output
        if (sub != 0) return;
        uint64_t* out = p.part + ((((size_t)l * B + b) * p.Hq + g * G + gi) * p.n_split + split) * (D + 2);
        if (cx.lane == 0) {
            st_tag(out + 0, 0.f, cx.epoch);
            st_tag(out + 1, 1.f, cx.epoch);
        }
#pragma unroll
        for (int h = 0; h < NH; ++h) st_tag(out + 2 + h * 64 + cx.lane, 0.f, cx.epoch);
        return;
    }

    const LDS float* qh = qs + gi * D;
    const float ninf = -__builtin_inff();
    float m = ninf, lsum = 0.f, o[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) o[h] = 0.f;
    const int od = ch * 8 + grp;  // the output dim (less 64 h) a lane's o[h] belongs to
    float4 qa[NH], qb[NH];  // the lane's q dims
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        qa[h] = lds_f4(qh + h * 64 + ch * 8);
        qb[h] = lds_f4(qh + h * 64 + ch * 8 + 4);
    }
    LDS float* eb = stt + NW * (D + 2) + cx.wave * 64;  // the wave's 64 softmax weights
    // PV of one 64-dim half: the lane's eight keys into its eight dims, then the reduce-scatter
    auto pv_half = [&](const uint4 (&r)[8], const float (&e8)[8], int nvalid) {
        float po[8];
#pragma unroll
        for (int d = 0; d < 8; ++d) po[d] = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            if (c * 8 >= nvalid) break;  // key group c lies past the split's keys
            const uint4 v = r[c];
            po[0] = fmaf(e8[c], bf_lo(v.x), po[0]);
            po[1] = fmaf(e8[c], bf_hi(v.x), po[1]);
            po[2] = fmaf(e8[c], bf_lo(v.y), po[2]);
            po[3] = fmaf(e8[c], bf_hi(v.y), po[3]);
            po[4] = fmaf(e8[c], bf_lo(v.z), po[4]);
            po[5] = fmaf(e8[c], bf_hi(v.z), po[5]);
            po[6] = fmaf(e8[c], bf_lo(v.w), po[6]);
            po[7] = fmaf(e8[c], bf_hi(v.w), po[7]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) po[i] = bfly<32>(po[i], po[i + 4], cx.lane);
#pragma unroll
        for (int i = 0; i < 2; ++i) po[i] = bfly<16>(po[i], po[i + 2], cx.lane);
        return bfly<8>(po[0], po[1], cx.lane);
    };
    for (int kb = sub; kb * 64 < nkeys; kb += wph) {
        const int kbase = j0 + kb * 64;
        const int rel = pos - kbase;
        const bool has_new = rel >= 0 && rel < 64 && pos < j1;  // uniform
        const bool has_next = (kb + wph) * 64 < nkeys;
        // keys of the block inside the split: with 128-dim heads the products of key groups c
        // with 8c >= nvalid (which hold none) are skipped, half the block at 32 keys per split;
        // with 64-dim heads the branches cost more than they save
        const int nvalid = NH == 2 ? min(64, nkeys - kb * 64) : 64;
        if (has_new) {
            put_new(kr, kn, rel);
            if constexpr (NH == 1) put_new(vr, vn, rel);
            else put_new(vr, kn + 64, rel);
        }
        float sp8[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            sp8[c] = 0.f;
            if (c * 8 < nvalid) {
                sp8[c] = dot8(kr[c], qa[0], qb[0]);
                if constexpr (NH == 2) sp8[c] += dot8(vr[c], qa[1], qb[1]);
            }
        }
        CBAR();  // the K tiles are consumed: their registers take the next loads
        if constexpr (NH == 1) {
            if (has_next) load_blk(kr, kres, kb + wph, 0);
        } else {
            load_blk(kr, vres, kb, 0);
            load_blk(vr, vres, kb, 1);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sp8[i] = bfly<4>(sp8[i], sp8[i + 4], cx.lane);
#pragma unroll
        for (int i = 0; i < 2; ++i) sp8[i] = bfly<2>(sp8[i], sp8[i + 2], cx.lane);
        // (every lane takes part in the exchange: a lane left out would hand its partner a
        // stale value)
        const float sfull = bfly<1>(sp8[0], sp8[1], cx.lane);
        const bool valid = kbase + od < j1;  // this lane's key is 8(L%8) + L/8, like its dim
        const float sc = valid ? sfull : ninf;
        const float mn = fmaxf(m, wave_max(sc));
        const float e = valid ? __expf(sc - mn) : 0.f;
        const float corr = m == ninf ? 0.f : __expf(m - mn);
        lsum = lsum * corr + wave_sum(e);
        m = mn;
        eb[cx.lane] = e;
        CBAR();  // a wave's LDS accesses complete in order: the reads below see all 64 writes
        const float4 ea = lds_f4(eb + grp * 8), ec = lds_f4(eb + grp * 8 + 4);
        const float e8[8] = {ea.x, ea.y, ea.z, ea.w, ec.x, ec.y, ec.z, ec.w};
        if constexpr (NH == 1) {
            o[0] = o[0] * corr + pv_half(vr, e8, nvalid);
            CBAR();
            if (has_next) load_blk(vr, vres, kb + wph, 0);
        } else {
            if (has_new) {
                put_new(kr, vn, rel);
                put_new(vr, vn + 64, rel);
            }
            o[0] = o[0] * corr + pv_half(kr, e8, nvalid);
            o[1] = o[1] * corr + pv_half(vr, e8, nvalid);
            CBAR();
            if (has_next) {
                load_blk(kr, kres, kb + wph, 0);
                load_blk(vr, kres, kb + wph, 1);
            }
        }
    }
    mark_mid(cx);
    const int head = g * G + gi;
    uint64_t* out = p.part + ((((size_t)l * B + b) * p.Hq + head) * p.n_split + split) * (D + 2);
    if (nkeys <= 64) {
        // one key block: the first wave of each head saw every key; it writes
        // the partial itself (no cross-wave merge)
        if (sub != 0 || cx.aborted) return;
        if (cx.lane == 0) {
            st_tag(out + 0, m, cx.epoch);
            st_tag(out + 1, lsum, cx.epoch);
        }
#pragma unroll
        for (int h = 0; h < NH; ++h) st_tag(out + 2 + h * 64 + od, o[h], cx.epoch);
        return;
    }
    // per-wave state -> LDS, merge the waves of each head
    LDS float* my = stt + cx.wave * (D + 2);
    if (cx.lane == 0) {
        my[0] = m;
        my[1] = lsum;
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) my[2 + h * 64 + od] = o[h];
    cbar(cx, s, seq);
    if (sub != 0 || cx.aborted) return;
    float M = ninf;
    for (int w = gi; w < NW; w += G) M = fmaxf(M, stt[w * (D + 2)]);
    float Ls = 0.f, O[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) O[h] = 0.f;
    if (M != ninf) {
        for (int w = gi; w < NW; w += G) {
            const LDS float* sw = stt + w * (D + 2);
            const float f = sw[0] == ninf ? 0.f : __expf(sw[0] - M);
            Ls = fmaf(sw[1], f, Ls);
#pragma unroll
            for (int h = 0; h < NH; ++h) O[h] = fmaf(sw[2 + h * 64 + cx.lane], f, O[h]);
        }
    }
    if (cx.lane == 0) {
        st_tag(out + 0, M, cx.epoch);
        st_tag(out + 1, Ls, cx.epoch);
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) st_tag(out + 2 + h * 64 + cx.lane, O[h], cx.epoch);
}



// Log-sum-exp merge of the n_split partials of (row b, head):
// out = sum_s o_s e^(m_s - M) / sum_s l_s e^(m_s - M), M = max_s m_s.
template <bool ABLATE>
__device__ __forceinline__ void op_reduce(Ctx& cx, const Lds& s, uint32_t r, const Inst& in, LDS float* xb) {
    CParams& p = *cx.p;
    const int B = p.B, D = p.D, l = in.layer, b = in.a, head = in.b, ns = p.n_split, W = D + 2;
    wait_inputs(cx, s, r);  // xb = the n_split partials, staged by the gather wave
    if (cx.wave != 0 || cx.aborted) return;
    if (ABLATE && p.ablate_op == OP_ATTN_REDUCE) {  // switched off: a zero output
        uint64_t* out = p.attn + ((size_t)l * B + b) * p.Hq * D + (size_t)head * D;
        for (int d = cx.lane; d < D; d += 64) st_tag(out + d, 0.f, cx.epoch);
        return;
    }
    const float ninf = -__builtin_inff();
    // the splits' (m, l) across lanes: M = max over splits, each split's weight
    // f_s = e^(m_s - M) (0 for a split without keys) replaces its m in LDS, Ls = sum of l_s f_s
    float M = ninf;
    for (int sp = cx.lane; sp < ns; sp += 64) M = fmaxf(M, xb[sp * W]);
    M = wave_max(M);
    float Ls = 0.f;
    for (int sp = cx.lane; sp < ns; sp += 64) {
        const float ms = xb[sp * W];
        const float f = ms == ninf ? 0.f : __expf(ms - M);
        Ls = fmaf(xb[sp * W + 1], f, Ls);
        xb[sp * W] = f;
    }
    Ls = wave_sum(Ls);
    CBAR();  // a wave's LDS accesses complete in order: the reads below see every weight
    // lane d owns dims d (and d + 64); the loop is unrolled so the LDS reads overlap
    const int nh = D / 64;
    float O0 = 0.f, O1 = 0.f;
    int sp = 0;
    for (; sp + 8 <= ns; sp += 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const LDS float* ps = xb + (sp + i) * W;
            const float f = ps[0];
            O0 = fmaf(ps[2 + cx.lane], f, O0);
            if (nh == 2) O1 = fmaf(ps[2 + 64 + cx.lane], f, O1);
        }
    }
    for (; sp < ns; ++sp) {
        const LDS float* ps = xb + sp * W;
        const float f = ps[0];
        O0 = fmaf(ps[2 + cx.lane], f, O0);
        if (nh == 2) O1 = fmaf(ps[2 + 64 + cx.lane], f, O1);
    }
    const float inv = 1.0f / Ls;
    uint64_t* out = p.attn + ((size_t)l * B + b) * p.Hq * D + (size_t)head * D;
    st_tag(out + cx.lane, O0 * inv, cx.epoch);
    if (nh == 2) st_tag(out + 64 + cx.lane, O1 * inv, cx.epoch);
}

// ---------------------------------------------------------- fused greedy --

__device__ __forceinline__ void argmax_pair(float& v, uint32_t& i, float ov, uint32_t oi) {
    if (ov > v || (ov == v && oi < i)) {
        v = ov;
        i = oi;
    }
}

// Greedy decoding inside the step (the single-launch GREEDY build): the LM-head epilogue keeps
// each CU's best row per batch row as an LDS key (greedy_key, LDS atomic max); after its queue,
// every CU publishes its (max, lowest index) pairs as tagged words; the last CU to count itself
// in (every other CU has then finished its queue, so none reads the tokens or positions any
// more) merges all pairs, one compute wave per batch row, writes next token = argmax of each
// logits row (lowest index among equal maxima, NaN never wins, 0 for a row without a number)
// and advances the positions, then resets the counter for the next launch.
__device__ __forceinline__ void greedy_finish(Ctx& cx, const Lds& s, const Step& sp, uint32_t& seq) {
    CParams& p = *cx.p;
    const int B = p.B;
    if (cx.aborted) return;
    cbar(cx, s, seq);  // every wave is past its last instruction (its key updates are applied)
    if (cx.aborted) return;
    if (cx.wave == 0) {
        if (cx.lane < B) {
            float v;
            uint32_t i;
            greedy_unkey(s.gkey[cx.lane], v, i);
            uint64_t* q = p.greedy_pair + ((size_t)cx.cu * MAX_BATCH + cx.lane) * 2;
            st_tag(q, v, cx.epoch);
            st_tag(q + 1, __uint_as_float(i), cx.epoch);
        }
        uint32_t old = 0;
        if (cx.lane == 0) old = __hip_atomic_fetch_add(p.greedy_cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = uni(old) == (uint32_t)p.ncu - 1;
        if (cx.lane == 0) {
            if (last) __hip_atomic_store(p.greedy_cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *s.glast = last ? 1u : 0u;
        }
    }
    cbar(cx, s, seq);
    if (cx.aborted || uni(lds_ld(s.glast)) == 0u || cx.wave >= B) return;
    // the last CU: compute wave bb merges batch row bb over every CU's pair, each lane polling four
    // CUs' pairs (value word and index word in one 16-byte load) at once
    const int bb = cx.wave, ncu = p.ncu;
    const uint32_t ep = cx.epoch;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.greedy_pair, (short)0, ncu * MAX_BATCH * 16, RSRC_WORD3);
    float bv = -__builtin_inff();
    uint32_t bi = GREEDY_NONE;
    for (int c0 = 0; c0 < ncu; c0 += 256) {
        u32x4 w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            w[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, ((c0 + 64 * j + cx.lane) * MAX_BATCH + bb) * 16, 0, CPOL_SC1);
        uint32_t spins = 0;
        while (true) {
            bool stale = false;
#pragma unroll
            for (int j = 0; j < 4; ++j) stale |= c0 + 64 * j + cx.lane < ncu && (w[j].y != ep || w[j].w != ep);
            if (!any_lane(stale)) break;
            if (!keep_waiting(cx, spins, 0x60000000u | (uint32_t)c0)) return;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = c0 + 64 * j + cx.lane;
                if (c < ncu && (w[j].y != ep || w[j].w != ep))
                    w[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (c * MAX_BATCH + bb) * 16, 0, CPOL_SC1);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (c0 + 64 * j + cx.lane < ncu) argmax_pair(bv, bi, __uint_as_float(w[j].x), w[j].z);
    }
    for (int d = 32; d >= 1; d >>= 1) {
        const float ov = __shfl_xor(bv, d);
        const uint32_t oi = (uint32_t)__shfl_xor((int)bi, d);
        argmax_pair(bv, bi, ov, oi);
    }
    if (cx.lane == 0) {
        gst((int32_t*)sp.tokens + bb, bi == GREEDY_NONE ? 0 : (int32_t)bi);
        gst((int32_t*)sp.positions + bb, __builtin_amdgcn_readlane(sp.pos, bb) + 1);
    }
}

// --------------------------------------------------------------- the kernel --

// stage < 0: run the whole queue (one launch per step); stage >= 0: only that
// stage's instructions (one launch per op and layer).  One instantiation per
// head size, each with and without the profile/timeline instrumentation (its
// bookkeeping costs registers and scalar work on every instruction, so the
// plain build leaves it out entirely).
template <int HEAD_DIM, bool INSTR, bool FP8, bool GREEDY, bool ABLATE>
__device__ __forceinline__ void step_body(const Params* __restrict__ pp, const int32_t* tokens,
                                          const int32_t* positions, uint16_t* kv, float* logits, int stage,
                                          uint32_t flags) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    CParams& p = *(CParams*)pp;
    Ctx cx;
    cx.p = (CParams*)pp;
    cx.cu = blockIdx.x;
    cx.lane = threadIdx.x & 63;
    const int wave = (int)uni(threadIdx.x >> 6);
    cx.aborted = false;
    cx.resident = stage < 0 && pp->res_stride > 0;
    cx.pc = 0;
    cx.op = 0;
    cx.slot = 0;
    cx.prof = INSTR && p.prof != nullptr;
    cx.trace = INSTR && p.trace != nullptr;
    cx.t_in = cx.t_acq = cx.t_mid = cx.t_ring = 0;
    for (int k = 0; k < 8; ++k) cx.cnt[k] = 0;
    const uint64_t t_kernel = cx.prof ? cycles() : 0;
    auto flush_prof = [&](int wave_slot) {
        if (cx.prof && cx.lane == 0) {
            GLB uint64_t* o = (GLB uint64_t*)p.prof + ((size_t)cx.cu * (NW + NLOAD) + wave_slot) * PROF_SLOTS;
            o[0] = cycles() - t_kernel;
            for (int k = 1; k < 8; ++k) o[k] = cx.cnt[k];
        }
    };
    cx.epoch = p.epoch[cx.cu] + 1;
    const Lds s = lds_map((LDS uint8_t*)smem, p);

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
    if (flags & KF_POISON) {  // debugging: every LDS word NaN until something writes it
        for (uint32_t i = threadIdx.x; i < p.lds_bytes / 4; i += WG_THREADS) ((LDS uint32_t*)smem)[i] = 0xffffffffu;
        __syncthreads();
    }
    if (threadIdx.x < SYNC_WORDS) s.landed[threadIdx.x] = 0;
    __syncthreads();

    const CONST_AS uint32_t* uoff = (const CONST_AS uint32_t*)(p.unit_off + ((size_t)qb + cx.cu) * NW);
    if (wave >= NW + NWL) {  // gather waves
        cx.wave = wave;
        gatherer<FP8>(cx, s, sp, qb, pc0, pc1, wave - NW - NWL);
        flush_prof(wave);
        return;
    }
    if (wave >= NW) {  // the weight loader of every compute wave
        cx.wave = wave;
        loader(cx, s, uoff, pc0, pc1);
        flush_prof(wave);
        return;
    }
    cx.wave = wave;
    Stream st{0, 0, 0, 0};
    uint32_t seq = 0;
    DownAcc da;
    for (int k = 0; k < DREG; ++k) da.r[k] = 0.f;
    // instructions are fetched one ahead so the fetch latency overlaps the
    // current instruction
    const CONST_AS u32x4* iq = (const CONST_AS u32x4*)(p.insts + uni(qb));
    u32x4 next = pc0 < pc1 ? iq[pc0] : u32x4{0, 0, 0, 0};
    const uint32_t nslot = uni((uint32_t)p.nslot);
    uint32_t slot = 0;  // buffer set of instruction pc (rotates with the gather wave's)
    for (uint32_t pc = pc0; pc < pc1 && !cx.aborted; ++pc, slot = slot + 1 == nslot ? 0 : slot + 1) {
        const u32x4 raw = next;
        if (pc + 1 < pc1) next = iq[pc + 1];
        Inst in;
        in.op = (uint16_t)(raw.x & 0xffffu);
        in.layer = (uint16_t)(raw.x >> 16);
        in.rg0 = raw.y;
        in.nrg = raw.z;
        in.a = (uint16_t)(raw.w & 0xffffu);
        in.b = (uint16_t)(raw.w >> 16);
        cx.pc = pc;
        cx.op = in.op;
        const uint64_t t_start = cx.trace ? rtime() : 0;
        cx.t_acq = cx.t_in = cx.t_mid = t_start;
        cx.t_ring = 0;
        const uint32_t r = pc - pc0;
        cx.slot = slot;
        LDS float* xb = xslot(s, p, slot);
        switch (in.op) {
        case OP_ATTENTION:
            op_attention_t<HEAD_DIM, ABLATE>(cx, s, seq, r, in, xb, sp);
            vm_drain();  // no load of the attention body stays tracked into the next instruction
            break;
        case OP_ATTN_REDUCE: op_reduce<ABLATE>(cx, s, r, in, xb); break;
        default: {
            const int ku = in.op == OP_O_PROJ_RES ? p.ku_q : in.op == OP_DOWN_RES ? p.ku_f : p.ku_h;
            if (!batch1_path(p.B, ku, FP8)) op_gemv<0, FP8, GREEDY, ABLATE>(cx, s, st, r, slot, in, xb, sp, da, seq);
            else if (!FP8 && ku == 4) op_gemv<FP8 ? 2 : 4, FP8, GREEDY, ABLATE>(cx, s, st, r, slot, in, xb, sp, da, seq);
            else op_gemv<2, FP8, GREEDY, ABLATE>(cx, s, st, r, slot, in, xb, sp, da, seq);
            break;
        }
        }
        // this wave is done with the instruction's staged inputs
        CBAR();
        if (cx.lane == 0) lds_st(s.done + wave, pc - pc0 + 1);
        if (cx.trace && cx.lane == 0) {
            GLB uint64_t* r = (GLB uint64_t*)p.trace + (size_t)(qb + pc) * TRACE_SLOTS;
            if (wave == 0)
                r[0] = (uint64_t)in.op | ((uint64_t)in.layer << 8) | ((uint64_t)in.a << 16) | ((uint64_t)in.b << 32) |
                       ((uint64_t)cx.cu << 48);
            GLB uint64_t* rw = r + 1 + TRACE_WAVE_SLOTS * wave;
            rw[0] = t_start;
            rw[1] = cx.t_acq;
            rw[2] = cx.t_in;
            rw[3] = cx.t_mid;
            rw[4] = rtime();
            rw[5] = cx.t_ring;
        }
    }
    if constexpr (GREEDY) greedy_finish(cx, s, sp, seq);
    flush_prof(wave);
    if ((flags & KF_BUMP_EPOCH) && wave == 0 && cx.lane == 0) p.epoch[cx.cu] = cx.epoch;
}

// The whole step in one launch (every workgroup runs its full queue); GREEDY: the build that
// also writes the argmax tokens and advances the positions; ABLATE: the build that can skip
// the arithmetic of one opcode (Params::ablate_op) while keeping its data flow.
// (BATCHED names the build in the kernel's symbol: the two builds of this file never share one)
template <int HEAD_DIM, bool INSTR, bool FP8 = false, bool GREEDY = false, bool ABLATE = false,
          bool BATCHED = TU_BATCHED>
__global__ void __launch_bounds__(WG_THREADS, 1)
mk_decode_kernel(const Params* __restrict__ pp, const int32_t* tokens, const int32_t* positions, uint16_t* kv,
                 float* logits, int stage, uint32_t flags) {
    step_body<HEAD_DIM, INSTR, FP8, GREEDY, ABLATE>(pp, tokens, positions, kv, logits, -1, flags);
}

// One stage of the step (one op of one layer) per launch.
template <int HEAD_DIM, bool INSTR, bool FP8 = false, bool BATCHED = TU_BATCHED>
__global__ void __launch_bounds__(WG_THREADS, 1)
mk_stage_kernel(const Params* __restrict__ pp, const int32_t* tokens, const int32_t* positions, uint16_t* kv,
                float* logits, int stage, uint32_t flags) {
    step_body<HEAD_DIM, INSTR, FP8, false, false>(pp, tokens, positions, kv, logits, stage, flags);
}

#if !MK_BATCHED_TU
// ----------------------------------------------------------- debug fill --

// The NaN fill of MK_FLAG_DEBUG_NAN before a step: the value half of every tagged word (its tag,
// a previous step's, stays), the down-projection accumulators and the logits.
__global__ void __launch_bounds__(256) mk_poison_kernel(uint64_t* arena, size_t words, float* f0, size_t n0,
                                                        float* f1, size_t n1) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride)
        arena[i] = (arena[i] & 0xffffffff00000000ull) | 0xffffffffull;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n0; i += stride) f0[i] = __int_as_float(-1);
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n1; i += stride) f1[i] = __int_as_float(-1);
}

hipError_t launch_poison(uint64_t* arena, size_t words, float* f0, size_t n0, float* f1, size_t n1,
                         hipStream_t stream) {
    hipLaunchKernelGGL(mk_poison_kernel, dim3(1024), dim3(256), 0, stream, arena, words, f0, n0, f1, n1);
    return hipGetLastError();
}

// ------------------------------------------------------------ pack kernel --

struct PackRowDev {
    uint32_t mat, row, k0, klen, src_cols, kunits, ustride, grow;
    uint64_t dst_unit;
};

// OCP E4M3 code of the value nearest to x (ties to the even mantissa), +-448
// for |x| >= 448: below 2^-6 the spacing is 2^-9 (subnormals, and 8 * 2^-9 is
// the smallest normal's code 0x08); above, the 23-bit fp32 mantissa is
// rounded to 3 bits.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const float a = fabsf(x);
    if (!(a < 448.f)) return sign | 0x7Eu;
    if (a < 0x1p-6f) return sign | (uint32_t)rintf(a * 512.f);
    int e = (int)((u >> 23) & 0xffu) - 127;  // -6 .. 8
    uint32_t q = (u >> 20) & 7u;
    const uint32_t low = u & 0xfffffu;
    if (low > 0x80000u || (low == 0x80000u && (q & 1u))) ++q;
    if (q == 8u) {
        q = 0;
        ++e;
    }
    if (e > 8 || (e == 8 && q == 7u)) return sign | 0x7Eu;
    return sign | ((uint32_t)(e + 7) << 3) | q;
}

// Largest |w| of each row of a [rows][cols] bf16 matrix, as bf16 bits (sign
// cleared: finite bf16 magnitudes order like their bits): one wave per row.
__global__ void __launch_bounds__(256) mk_row_amax_kernel(const uint16_t* w, uint32_t rows, uint32_t cols,
                                                          uint16_t* out) {
    const uint32_t lane = threadIdx.x & 63, nw = gridDim.x * (blockDim.x >> 6);
    for (uint32_t r = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); r < rows; r += nw) {
        const uint16_t* row = w + (size_t)r * cols;
        uint32_t m = 0;
        for (uint32_t c = lane; c < cols; c += 64) {
            const uint32_t v = row[c] & 0x7fffu;
            m = v > m ? v : m;
        }
        for (int d = 32; d >= 1; d >>= 1) {
            const uint32_t o = (uint32_t)__shfl_xor((int)m, d);
            m = o > m ? o : m;
        }
        if (lane == 0) out[r] = (uint16_t)m;
    }
}

// One workgroup per stream row: dst[unit .. unit + kunits) = src row slice, zero padded;
// with fp8, the codes of fp32(w / scale[row]) (1024 per unit) instead of the bf16 values.
__global__ void __launch_bounds__(256) mk_pack_kernel(const PackRowDev* rows, uint32_t n, const uint16_t* const* mats,
                                                      uint8_t* dst, int fp8, const float* scales) {
    for (uint32_t r = blockIdx.x; r < n; r += gridDim.x) {
        const PackRowDev pr = rows[r];
        if (fp8) {
            const uint16_t* src = mats[pr.mat] + (size_t)pr.row * pr.src_cols + pr.k0;
            const float sc = scales[pr.grow];
            const uint32_t n_el = pr.kunits * FP8_UNIT_ELEMS;
            for (uint32_t e = threadIdx.x; e < n_el; e += blockDim.x) {
                uint8_t* out = dst + (pr.dst_unit + (uint64_t)(e / FP8_UNIT_ELEMS) * NW * pr.ustride) * UNIT_BYTES;
                out[e % FP8_UNIT_ELEMS] = e < pr.klen ? (uint8_t)e4m3_code(bf2f(src[e]) / sc) : (uint8_t)0;
            }
            continue;
        }
        const uint16_t* src = mats[pr.mat] + (size_t)pr.row * pr.src_cols + pr.k0;
        const uint32_t n_el = pr.kunits * UNIT_ELEMS;
        for (uint32_t e = threadIdx.x; e < n_el; e += blockDim.x) {
            // element e lies in the row's unit e / 512, and consecutive units of a
            // stream are NW units apart in the packed buffer
            uint16_t* out =
                (uint16_t*)(dst + (pr.dst_unit + (uint64_t)(e / UNIT_ELEMS) * NW * pr.ustride) * UNIT_BYTES);
            out[e % UNIT_ELEMS] = e < pr.klen ? src[e] : (uint16_t)0;
        }
    }
}

// ------------------------------------------------------------ greedy step --

// tokens[b] = argmax_v logits[b][v] (lowest index among equal maxima, NaN
// never wins, an all-NaN row gives 0), positions[b] += 1.  GREEDY_BLOCKS
// workgroups share a row: each reduces its slice to a (value, index) pair,
// and the last one to finish (a device-scope counter per row) reduces the
// pairs and writes the token.  The counter is reset by that last workgroup,
// so the next call starts from zero.
constexpr int GREEDY_THREADS = 256;
struct ArgMax {
    float v;
    int i;
};
__device__ __forceinline__ void argmax_take(ArgMax& a, float v, int i) {
    if (v > a.v || (v == a.v && i < a.i)) {
        a.v = v;
        a.i = i;
    }
}
__device__ __forceinline__ ArgMax argmax_block(ArgMax a, ArgMax* sh) {
    for (int off = 32; off >= 1; off >>= 1) argmax_take(a, __shfl_xor(a.v, off), __shfl_xor(a.i, off));
    const int t = threadIdx.x;
    if ((t & 63) == 0) sh[t >> 6] = a;
    __syncthreads();
    if (t == 0)
        for (int w = 1; w < GREEDY_THREADS / 64; ++w) argmax_take(a, sh[w].v, sh[w].i);
    return a;  // complete in thread 0
}
__global__ void __launch_bounds__(GREEDY_THREADS) mk_greedy_kernel(const float* logits, int V, int32_t* tokens,
                                                                    int32_t* positions, uint64_t* part, uint32_t* cnt) {
    __shared__ ArgMax sh[GREEDY_THREADS / 64];
    __shared__ bool last;
    const int b = blockIdx.y, blk = blockIdx.x, nb = gridDim.x, t = threadIdx.x;
    const float* row = logits + (size_t)b * V;
    // slice [v0, v1), 4-aligned when the row is 16-byte aligned
    const int per = ((V + nb - 1) / nb + 3) & ~3;
    const int v0 = blk * per < V ? blk * per : V, v1 = v0 + per < V ? v0 + per : V;
    ArgMax a{-__builtin_inff(), 0x7fffffff};
    const bool vec = ((uintptr_t)row & 15) == 0;
    const int n4 = vec ? (v1 - v0) / 4 : 0;
    for (int c = t; c < n4; c += GREEDY_THREADS) {
        const f32x4 x = *(const GLB f32x4*)(row + v0 + 4 * c);
        const int i = v0 + 4 * c;
        argmax_take(a, x.x, i);
        argmax_take(a, x.y, i + 1);
        argmax_take(a, x.z, i + 2);
        argmax_take(a, x.w, i + 3);
    }
    for (int i = v0 + 4 * n4 + t; i < v1; i += GREEDY_THREADS) argmax_take(a, gld(row + i), i);
    a = argmax_block(a, sh);
    if (t == 0) {
        __hip_atomic_store((GLB uint64_t*)&part[(size_t)b * nb + blk], ((uint64_t)(uint32_t)a.i << 32) | __float_as_uint(a.v),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the pair is ordered before the count (release); the last arrival
        // orders its reads after it (acquire)
        const uint32_t old = __hip_atomic_fetch_add(&cnt[b], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        last = old == (uint32_t)nb - 1;
    }
    __syncthreads();
    if (!last) return;
    ArgMax f{-__builtin_inff(), 0x7fffffff};
    for (int k = t; k < nb; k += GREEDY_THREADS) {
        const uint64_t w = __hip_atomic_load((GLB uint64_t*)&part[(size_t)b * nb + k], __ATOMIC_ACQUIRE,
                                             __HIP_MEMORY_SCOPE_AGENT);
        argmax_take(f, __uint_as_float((uint32_t)w), (int)(w >> 32));
    }
    __syncthreads();
    f = argmax_block(f, sh);
    if (t == 0) {
        tokens[b] = f.i == 0x7fffffff ? 0 : f.i;
        positions[b] += 1;
        __hip_atomic_store(&cnt[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

hipError_t launch_greedy(const float* logits, int B, int V, int32_t* tokens, int32_t* positions, uint64_t* part,
                         uint32_t* cnt, hipStream_t stream) {
    hipLaunchKernelGGL(mk_greedy_kernel, dim3(GREEDY_BLOCKS, B), dim3(GREEDY_THREADS), 0, stream, logits, V, tokens,
                       positions, part, cnt);
    return hipGetLastError();
}

// ------------------------------------------------------------ litmus ------

// Litmus test of the tagged-word protocol and ping-pong latency probe.  Pair
// p is workgroup p (ping) and workgroup npairs + p (pong); with round-robin
// dispatch over the XCDs the two share an XCD exactly when npairs is a
// multiple of their number.  In round r the ping writes `words` tagged words
// {value f(p, r, k), tag r + 1} with the same agent-coherent stores as the
// step kernel; the pong polls them with the same loads until every tag is
// r + 1, checks every value that arrived with the tag, and answers with
// {g(p, r, k), r + 1}, which the ping polls and checks before its next round.
// A value that is not the one stored with its tag counts as a mismatch; a
// poll that exceeds spin_limit counts as a timeout and ends the pair's run.
// result: [0] mismatches, [1] timeouts, [2] completed round trips, then per
// pair [3 + 3p] ticks of the 100 MHz clock the ping spent, [4 + 3p] ping XCC,
// [5 + 3p] pong XCC.
__device__ __forceinline__ uint32_t litmus_value(uint32_t pair, uint32_t r, uint32_t k, uint32_t dir) {
    uint32_t x = pair * 0x9E3779B1u ^ (r + 1u) * 0x85EBCA77u ^ k * 0xC2B2AE3Du ^ dir * 0x27D4EB2Fu;
    x ^= x >> 15;
    x *= 0x2C1B3C6Du;
    x ^= x >> 12;
    return x;
}
__device__ __forceinline__ uint32_t xcc_id() {
    // HW_REG_XCC_ID (hardware register 20), bits 3:0
    return (uint32_t)__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xfu;
}
constexpr int LITMUS_MAX_WORDS = 1024;  // 16 words per lane
__global__ void __launch_bounds__(64) mk_litmus_kernel(uint64_t* buf, int npairs, int rounds, int words,
                                                       uint32_t spin_limit, uint32_t* result) {
    const int wg = blockIdx.x, lane = threadIdx.x;
    const bool ping = wg < npairs;
    const uint32_t pair = (uint32_t)(ping ? wg : wg - npairs);
    uint64_t* fwd = buf + (size_t)pair * 2 * words;  // ping -> pong
    uint64_t* back = fwd + words;                    // pong -> ping
    uint32_t mism = 0, timeouts = 0, done = 0;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    auto send = [&](uint64_t* dst, uint32_t r, uint32_t dir) {
        for (int k = lane; k < words; k += 64) st_tag(dst + k, __uint_as_float(litmus_value(pair, r, k, dir)), r + 1u);
    };
    // polls src until every tag is r + 1; false on timeout
    auto recv = [&](const uint64_t* src, uint32_t r, uint32_t dir) -> bool {
        uint64_t w[LITMUS_MAX_WORDS / 64];
#pragma unroll
        for (int j = 0; j < LITMUS_MAX_WORDS / 64; ++j) w[j] = lane + 64 * j < words ? ld_tag(src + lane + 64 * j) : 0;
        uint32_t spins = 0;
        while (true) {
            bool stale = false;
#pragma unroll
            for (int j = 0; j < LITMUS_MAX_WORDS / 64; ++j) stale |= lane + 64 * j < words && tag_of(w[j]) != r + 1u;
            if (!any_lane(stale)) break;
            if (++spins > spin_limit) return false;
            __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int j = 0; j < LITMUS_MAX_WORDS / 64; ++j)
                if (lane + 64 * j < words && tag_of(w[j]) != r + 1u) w[j] = ld_tag(src + lane + 64 * j);
        }
#pragma unroll
        for (int j = 0; j < LITMUS_MAX_WORDS / 64; ++j)
            if (lane + 64 * j < words && __float_as_uint(val_of(w[j])) != litmus_value(pair, r, lane + 64 * j, dir)) ++mism;
        return true;
    };
    for (int r = 0; r < rounds; ++r) {
        if (ping) {
            send(fwd, (uint32_t)r, 0);
            if (!recv(back, (uint32_t)r, 1)) { ++timeouts; break; }
        } else {
            if (!recv(fwd, (uint32_t)r, 0)) { ++timeouts; break; }
            send(back, (uint32_t)r, 1);
        }
        ++done;
    }
    const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
    for (int o = 32; o >= 1; o >>= 1) mism += (uint32_t)__shfl_xor((int)mism, o);
    if (lane == 0) {
        atomicAdd(&result[0], mism);
        atomicAdd(&result[1], uni(timeouts));
        if (ping) {
            atomicAdd(&result[2], done);
            result[3 + 3 * pair] = (uint32_t)(t1 - t0);
            result[4 + 3 * pair] = xcc_id();
        } else {
            result[5 + 3 * pair] = xcc_id();
        }
    }
}

hipError_t launch_litmus(uint64_t* buf, int npairs, int rounds, int words, uint32_t spin_limit, uint32_t* result,
                         hipStream_t stream) {
    void* args[] = {(void*)&buf, (void*)&npairs, (void*)&rounds, (void*)&words, (void*)&spin_limit, (void*)&result};
    // every pair waits on its partner: the grid must be resident at once
    return hipLaunchCooperativeKernel((const void*)mk_litmus_kernel, dim3(2 * npairs), dim3(64), args, 0, stream);
}

// ------------------------------------------------------------ read probe --

// Streams `bytes` from buf once (16-byte loads, eight in flight per lane): the
// achievable HBM read rate that a step's weight stream competes for.
__global__ void __launch_bounds__(512) mk_read_probe_kernel(const uint8_t* buf, size_t bytes, uint32_t* sink) {
    const size_t n16 = bytes / 16;
    const size_t nthreads = (size_t)gridDim.x * blockDim.x;
    const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    // thread t reads chunks t, t + nthreads, ...: every wave reads 1 KiB contiguous per load
    uint32_t acc = 0;
    size_t i = t;
    for (; i + 7 * nthreads < n16; i += 8 * nthreads) {
        u32x4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = *(const GLB u32x4*)(buf + (i + k * nthreads) * 16);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    for (; i < n16; i += nthreads) {
        const u32x4 v = *(const GLB u32x4*)(buf + i * 16);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;  // keeps the loads; practically never taken
}

// A kernel that does nothing: the launch and dispatch cost alone.
__global__ void __launch_bounds__(1024) mk_empty_kernel() {}

hipError_t launch_empty(int n_blocks, int n_threads, hipStream_t stream) {
    hipLaunchKernelGGL(mk_empty_kernel, dim3(n_blocks), dim3(n_threads), 0, stream);
    return hipGetLastError();
}

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, int ncu, hipStream_t stream) {
    hipLaunchKernelGGL(mk_read_probe_kernel, dim3(ncu * 4), dim3(512), 0, stream, (const uint8_t*)buf, bytes, sink);
    return hipGetLastError();
}

// ------------------------------------------------------------ host launch --

#endif  // !MK_BATCHED_TU

#if MK_BATCHED_TU
#define MK_LAUNCH_STEP launch_step_batched
#define MK_SET_STEP_LDS set_step_kernel_lds_batched
#else
#define MK_LAUNCH_STEP launch_step_single
#define MK_SET_STEP_LDS set_step_kernel_lds_single
#endif
hipError_t launch_step_batched(const Params*, int, int, size_t, const int32_t*, const int32_t*, void*, float*, int,
                               uint32_t, hipStream_t);
hipError_t launch_step_single(const Params*, int, int, size_t, const int32_t*, const int32_t*, void*, float*, int,
                              uint32_t, hipStream_t);
hipError_t set_step_kernel_lds_batched(size_t);
hipError_t set_step_kernel_lds_single(size_t);

// The whole-step launch waits across workgroups, so it needs every workgroup
// resident at once: a cooperative launch guarantees that (or fails).  Per-op
// launches only read results of earlier launches and use an ordinary launch.
// (this build's step kernels: batch-1 or batched)
hipError_t MK_LAUNCH_STEP(const Params* dev_params, int head_dim, int ncu, size_t lds_bytes, const int32_t* tokens,
                          const int32_t* positions, void* kv, float* logits, int stage, uint32_t flags,
                          hipStream_t stream) {
    uint16_t* kv16 = (uint16_t*)kv;
    void* args[] = {(void*)&dev_params, (void*)&tokens, (void*)&positions, (void*)&kv16, (void*)&logits,
                    (void*)&stage, (void*)&flags};
    const bool instr = (flags & KF_INSTRUMENTED) != 0, fp8 = (flags & KF_FP8) != 0;
    if (fp8 && instr) return hipErrorInvalidValue;  // no instrumented FP8 build
    if (flags & KF_ABLATE) {  // single launch, bf16 plain builds only
        if (stage >= 0 || instr || fp8 || (flags & KF_GREEDY)) return hipErrorInvalidValue;
        const void* fn = head_dim == 64 ? (const void*)mk_decode_kernel<64, false, false, false, true>
                                        : (const void*)mk_decode_kernel<128, false, false, false, true>;
        return hipLaunchCooperativeKernel(fn, dim3(ncu), dim3(WG_THREADS), args, (unsigned)lds_bytes, stream);
    }
    if (flags & KF_GREEDY) {  // single launch, plain builds only
        if (stage >= 0 || instr) return hipErrorInvalidValue;
        const void* fn = fp8 ? (head_dim == 64 ? (const void*)mk_decode_kernel<64, false, true, true>
                                               : (const void*)mk_decode_kernel<128, false, true, true>)
                             : (head_dim == 64 ? (const void*)mk_decode_kernel<64, false, false, true>
                                               : (const void*)mk_decode_kernel<128, false, false, true>);
        return hipLaunchCooperativeKernel(fn, dim3(ncu), dim3(WG_THREADS), args, (unsigned)lds_bytes, stream);
    }
    if (stage < 0) {
        const void* fn =
            fp8 ? (head_dim == 64 ? (const void*)mk_decode_kernel<64, false, true> : (const void*)mk_decode_kernel<128, false, true>)
            : head_dim == 64 ? (instr ? (const void*)mk_decode_kernel<64, true> : (const void*)mk_decode_kernel<64, false>)
                             : (instr ? (const void*)mk_decode_kernel<128, true> : (const void*)mk_decode_kernel<128, false>);
        return hipLaunchCooperativeKernel(fn, dim3(ncu), dim3(WG_THREADS), args, (unsigned)lds_bytes, stream);
    }
    const void* fn =
        fp8 ? (head_dim == 64 ? (const void*)mk_stage_kernel<64, false, true> : (const void*)mk_stage_kernel<128, false, true>)
        : head_dim == 64 ? (instr ? (const void*)mk_stage_kernel<64, true> : (const void*)mk_stage_kernel<64, false>)
                         : (instr ? (const void*)mk_stage_kernel<128, true> : (const void*)mk_stage_kernel<128, false>);
    return hipLaunchKernel(fn, dim3(ncu), dim3(WG_THREADS), args, lds_bytes, stream);
}

hipError_t MK_SET_STEP_LDS(size_t lds_bytes) {
    const void* fns[] = {(const void*)mk_decode_kernel<64, false>, (const void*)mk_decode_kernel<128, false>,
                         (const void*)mk_stage_kernel<64, false>,  (const void*)mk_stage_kernel<128, false>,
                         (const void*)mk_decode_kernel<64, true>,  (const void*)mk_decode_kernel<128, true>,
                         (const void*)mk_stage_kernel<64, true>,   (const void*)mk_stage_kernel<128, true>,
                         (const void*)mk_decode_kernel<64, false, true>, (const void*)mk_decode_kernel<128, false, true>,
                         (const void*)mk_stage_kernel<64, false, true>,  (const void*)mk_stage_kernel<128, false, true>,
                         (const void*)mk_decode_kernel<64, false, false, true>, (const void*)mk_decode_kernel<128, false, false, true>,
                         (const void*)mk_decode_kernel<64, false, true, true>, (const void*)mk_decode_kernel<128, false, true, true>,
                         (const void*)mk_decode_kernel<64, false, false, false, true>,
                         (const void*)mk_decode_kernel<128, false, false, false, true>};
    for (const void* fn : fns) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

#if !MK_BATCHED_TU
// handles with several batch rows run the batched build (KF_BATCHED), batch-1 handles the other
hipError_t launch_step(const Params* dev_params, int head_dim, int ncu, size_t lds_bytes, const int32_t* tokens,
                       const int32_t* positions, void* kv, float* logits, int stage, uint32_t flags,
                       hipStream_t stream) {
    return (flags & KF_BATCHED ? launch_step_batched : launch_step_single)(
        dev_params, head_dim, ncu, lds_bytes, tokens, positions, kv, logits, stage, flags, stream);
}
hipError_t set_step_kernel_lds(size_t lds_bytes) {
    const hipError_t e = set_step_kernel_lds_single(lds_bytes);
    return e != hipSuccess ? e : set_step_kernel_lds_batched(lds_bytes);
}

hipError_t launch_pack(const void* rows, uint32_t n, const uint16_t* const* mats, uint8_t* dst, int fp8,
                       const float* scales, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const uint32_t grid = n < 65536 ? n : 65536;
    hipLaunchKernelGGL(mk_pack_kernel, dim3(grid), dim3(256), 0, stream, (const PackRowDev*)rows, n, mats, dst, fp8,
                       scales);
    return hipGetLastError();
}

hipError_t launch_row_amax(const uint16_t* w, uint32_t rows, uint32_t cols, uint16_t* out, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    const uint32_t blocks = (rows + 3) / 4;
    hipLaunchKernelGGL(mk_row_amax_kernel, dim3(blocks < 8192 ? blocks : 8192u), dim3(256), 0, stream, w, rows, cols,
                       out);
    return hipGetLastError();
}

#endif  // !MK_BATCHED_TU

}  // namespace mk
