// Batched prefill: one forward pass over every position of a prompt that
// fills the KV cache and yields the logits of the last position.  The opening
// section of "One Token, 2,400 Kernel Launches" contrasts this phase (the
// whole prompt at once, compute-saturated) with token-by-token decode; the
// math per position is the same Llama layer as the decode step, so the result
// equals running the decode step at positions 0 .. P-1 with the prompt tokens
// (up to fp32 rounding order).
//
// Rows are (batch row, position) pairs, so every projection is a dense
// contraction C[M][N] = A[M][K] * W[N][K]^T with M = B * P: those run on the
// bf16 matrix cores (fp32 activations as two bf16 terms against the bf16
// weights, fp32 sums; see gemm).  RMSNorm, RoPE + cache append, causal attention and
// SwiGLU are small vector kernels between them, all on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <algorithm>
#include <mutex>
#include "mk_internal.h"

namespace mk {
namespace pf {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN
__device__ __forceinline__ uint16_t to_bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float wsum(float x) {
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}
__device__ __forceinline__ float wmax(float x) {
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

// X[m][:] = E[token of row m], row m = b * Pc + (t - t0) of the chunk; an id
// outside [0, V) gives a zero row and is reported (*bad, and the device error
// record as a decode step reports one: code 2, detail the batch row)
__global__ void __launch_bounds__(256) embed(const int32_t* tokens, int P, int t0, int Pc, int H, int V,
                                             const uint16_t* E, float* X, uint32_t* bad, uint32_t* err) {
    const int m = blockIdx.x, b = m / Pc, t = t0 + m % Pc;
    int tk = tokens[(size_t)b * P + t];
    if (tk < 0 || tk >= V) {
        if (threadIdx.x == 0) {
            if (bad) atomicOr(bad, 1u);
            if (err) {
                if (atomicCAS(&err[0], 0u, 2u) == 0u) {
                    err[1] = 0xffffffffu;  // no workgroup of a decode step
                    err[2] = (uint32_t)t;
                    err[3] = 0u;
                    err[4] = 0u;
                    err[5] = (uint32_t)b;
                }
                atomicOr(&err[7], 1u);
            }
        }
        tk = -1;
    }
    for (int i = threadIdx.x; i < H; i += blockDim.x)
        X[(size_t)m * H + i] = tk < 0 ? 0.f : bf(E[(size_t)tk * H + i]);
}

// A[r][:] = X[r][:] * rsqrt(mean(X[r]^2) + eps) * gain, one row per block
__global__ void __launch_bounds__(256) rmsnorm(const float* X, size_t ldx, int H, const uint16_t* gain, float eps,
                                               float* A, size_t lda) {
    __shared__ float red[4];
    const float* x = X + (size_t)blockIdx.x * ldx;
    float ss = 0.f;
    for (int i = threadIdx.x; i < H; i += 256) ss += x[i] * x[i];
    ss = wsum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float sc = rsqrtf((red[0] + red[1] + red[2] + red[3]) * (1.0f / (float)H) + eps);
    float* a = A + (size_t)blockIdx.x * lda;
    for (int i = threadIdx.x; i < H; i += 256) a[i] = x[i] * sc * bf(gain[i]);
}

// C[M][N] (row stride ldc) = or += A[M][K] (stride lda) * W[N][K]^T.
// 64 x 64 tile per block of 4 waves, each wave a 32 x 32 quarter as 2 x 2
// C[M][N] (=, or += with accumulate) A[M][K] * W[N][K]^T on the bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16).  The fp32 activations go in as two bf16 terms,
// a = hi + lo with hi = bf16(a) and lo = bf16(a - hi) (16 significant bits), so
// every product with the bf16 weights is exact and the sums are fp32: two
// MFMAs per step.  Block tile 128 x 128 (four waves of 64 x 64, i.e. 4 x 4
// MFMA tiles each), K in steps of 32 staged through double-buffered LDS; the
// next step's global loads are in flight during the current step's MFMAs.
// K, lda and the pointers are multiples of 8 elements (the config guarantees
// it), so the staging loads are whole float4 / 8 x bf16 vectors, inside or
// outside K.  Operand layout (16x16x32): lane l holds A[l % 16][8 (l / 16) + j]
// and B[8 (l / 16) + j][l % 16], j < 8; the result's lane l holds rows
// 4 (l / 16) + i of column l % 16, i < 4.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
constexpr int BM = 128, BN = 128, BK = 32, LDK = BK + 8;  // LDS rows of 80 bytes: 16-byte aligned, banks staggered
__global__ void __launch_bounds__(256) gemm(const float* A, int lda, const uint16_t* W, int K, float* C, int ldc,
                                            int M, int N, int accumulate) {
    __shared__ __attribute__((aligned(16))) __bf16 Ah[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) __bf16 Al[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[2][BN * LDK];
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const int lr = lane & 15, lk = 8 * (lane >> 4);
    f32x4 acc[4][4];
    for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // staging: A is 128 rows x 8 float4 (four per thread), W 128 rows x 4 vectors of 8 bf16 (two)
    float4 ra[4];
    uint4 rw[2];
    auto gload = [&](int k0) {
        for (int i = 0; i < 4; ++i) {
            const int e = tid + i * 256, r = e >> 3, c = (e & 7) * 4, gm = m0 + r, gk = k0 + c;
            ra[i] = gm < M && gk < K ? *(const float4*)(A + (size_t)gm * lda + gk) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        for (int i = 0; i < 2; ++i) {
            const int e = tid + i * 256, r = e >> 2, c = (e & 3) * 8, gn = n0 + r, gk = k0 + c;
            rw[i] = gn < N && gk < K ? *(const uint4*)(W + (size_t)gn * K + gk) : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto sstore = [&](int buf) {
        for (int i = 0; i < 4; ++i) {
            const int e = tid + i * 256, r = e >> 3, c = (e & 7) * 4;
            const f32x4v x = {ra[i].x, ra[i].y, ra[i].z, ra[i].w};
            const bf16x4 hi = __builtin_convertvector(x, bf16x4);  // round to nearest even
            const bf16x4 lo = __builtin_convertvector(x - __builtin_convertvector(hi, f32x4v), bf16x4);
            *(bf16x4*)&Ah[buf][r * LDK + c] = hi;
            *(bf16x4*)&Al[buf][r * LDK + c] = lo;
        }
        for (int i = 0; i < 2; ++i) {
            const int e = tid + i * 256, r = e >> 2, c = (e & 3) * 8;
            *(uint4*)&Ws[buf][r * LDK + c] = rw[i];
        }
    };
    gload(0);
    sstore(0);
    __syncthreads();
    for (int k0 = 0, buf = 0; k0 < K; k0 += BK, buf ^= 1) {
        const bool more = k0 + BK < K;
        if (more) gload(k0 + BK);
        bf16x8 b[4];
        for (int tj = 0; tj < 4; ++tj) b[tj] = *(const bf16x8*)&Ws[buf][(wn + tj * 16 + lr) * LDK + lk];
        for (int ti = 0; ti < 4; ++ti) {
            const bf16x8 ah = *(const bf16x8*)&Ah[buf][(wm + ti * 16 + lr) * LDK + lk];
            const bf16x8 al = *(const bf16x8*)&Al[buf][(wm + ti * 16 + lr) * LDK + lk];
            for (int tj = 0; tj < 4; ++tj) {
                acc[ti][tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b[tj], acc[ti][tj], 0, 0, 0);
                acc[ti][tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b[tj], acc[ti][tj], 0, 0, 0);
            }
        }
        if (more) sstore(buf ^ 1);  // the other buffer was last read before the previous barrier
        __syncthreads();
    }
    for (int ti = 0; ti < 4; ++ti)
        for (int tj = 0; tj < 4; ++tj)
            for (int j = 0; j < 4; ++j) {
                const int r = m0 + wm + ti * 16 + 4 * (lane >> 4) + j, c = n0 + wn + tj * 16 + lr;
                if (r < M && c < N) {
                    float* p = C + (size_t)r * ldc + c;
                    *p = accumulate ? *p + acc[ti][tj][j] : acc[ti][tj][j];
                }
            }
}

// Row m = b * Pc + (t - t0) of QKV ([q heads | k heads | v heads], fp32): RoPE
// on the q and k heads at position t (rotate-half pairs, cos/sin from the handle's
// table), then k and v rounded to bf16 into cache slot t of layer `layer`.
__global__ void __launch_bounds__(256) rope_kv(float* QKV, int ld, int B, int t0, int Pc, int Hq, int Hkv, int D,
                                               const float* rope, uint16_t* kv, int layer, int max_seq) {
    const int m = blockIdx.x, b = m / Pc, t = t0 + m % Pc, half = D / 2;
    float* row = QKV + (size_t)m * ld;
    const int QD = Hq * D, KD = Hkv * D;
    for (int e = threadIdx.x; e < (Hq + Hkv) * half; e += 256) {
        const int head = e / half, i = e % half;
        float* x = row + (size_t)head * D;
        const float c = rope[((size_t)t * half + i) * 2], s = rope[((size_t)t * half + i) * 2 + 1];
        const float u = x[i], w = x[i + half];
        x[i] = u * c - w * s;
        x[i + half] = w * c + u * s;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < KD; e += 256) {
        const int g = e / D, d = e % D;
        const size_t kslot = ((((size_t)layer * 2 + 0) * B + b) * Hkv + g) * (size_t)max_seq + t;
        const size_t vslot = ((((size_t)layer * 2 + 1) * B + b) * Hkv + g) * (size_t)max_seq + t;
        kv[kslot * D + d] = to_bf(row[QD + e]);
        kv[vslot * D + d] = to_bf(row[QD + KD + e]);
    }
}

// Causal attention of query (row m of the chunk, head h) over cache slots
// 0 .. t of its KV group (earlier chunks' slots were written by their passes): one wave each, keys in blocks of 64 (lane j scores key j of the
// block), online softmax across blocks, lane d accumulating output dims
// d, d + 64.  O[m][h * D + d] = sum_j softmax(q . k_j / sqrt(D))_j v_j[d].
template <int D>
__global__ void __launch_bounds__(256) attention(const float* QKV, int ld, const uint16_t* kv, int B, int t0, int Pc,
                                                 int Hq, int Hkv, int layer, int max_seq, float* O, int ldo) {
    constexpr int NC = D / 64;
    __shared__ float qs[4][D];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wid = blockIdx.x * 4 + w;
    if (wid >= B * Pc * Hq) return;  // the whole wave leaves; no block barrier follows
    const int head = wid % Hq, m = wid / Hq, b = m / Pc, t = t0 + m % Pc, g = head / (Hq / Hkv);
    const float* q = QKV + (size_t)m * ld + (size_t)head * D;
    for (int d = lane; d < D; d += 64) qs[w][d] = q[d];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const uint16_t* Kb = kv + ((((size_t)layer * 2 + 0) * B + b) * Hkv + g) * (size_t)max_seq * D;
    const uint16_t* Vb = kv + ((((size_t)layer * 2 + 1) * B + b) * Hkv + g) * (size_t)max_seq * D;
    const float scale = rsqrtf((float)D);
    float mx = -__builtin_inff(), l = 0.f, o[NC];
    for (int c = 0; c < NC; ++c) o[c] = 0.f;
    for (int j0 = 0; j0 <= t; j0 += 64) {
        const int j = j0 + lane;
        float s = -__builtin_inff();
        if (j <= t) {
            const uint4* kr = (const uint4*)(Kb + (size_t)j * D);
            float acc = 0.f;
            for (int u = 0; u < D / 8; ++u) {
                const uint4 v = kr[u];
                const float* qq = &qs[w][u * 8];
                acc = fmaf(__uint_as_float(v.x << 16), qq[0], acc);
                acc = fmaf(__uint_as_float(v.x & 0xffff0000u), qq[1], acc);
                acc = fmaf(__uint_as_float(v.y << 16), qq[2], acc);
                acc = fmaf(__uint_as_float(v.y & 0xffff0000u), qq[3], acc);
                acc = fmaf(__uint_as_float(v.z << 16), qq[4], acc);
                acc = fmaf(__uint_as_float(v.z & 0xffff0000u), qq[5], acc);
                acc = fmaf(__uint_as_float(v.w << 16), qq[6], acc);
                acc = fmaf(__uint_as_float(v.w & 0xffff0000u), qq[7], acc);
            }
            s = acc * scale;
        }
        const float nm = fmaxf(mx, wmax(s));  // lane 0's key j0 <= t, so nm is finite
        const float p = j <= t ? __expf(s - nm) : 0.f;
        const float corr = __expf(mx - nm);
        l = l * corr + wsum(p);
        for (int c = 0; c < NC; ++c) o[c] *= corr;
        const int nk = t - j0 + 1 < 64 ? t - j0 + 1 : 64;
        for (int jj = 0; jj < nk; ++jj) {
            const float pj = __shfl(p, jj);
            const uint16_t* vr = Vb + (size_t)(j0 + jj) * D;
            for (int c = 0; c < NC; ++c) o[c] = fmaf(pj, bf(vr[lane + 64 * c]), o[c]);
        }
        mx = nm;
    }
    const float inv = 1.0f / l;
    for (int c = 0; c < NC; ++c) O[(size_t)m * ldo + (size_t)head * D + lane + 64 * c] = o[c] * inv;
}

// G[i] = silu(G[i]) * U[i]
__global__ void __launch_bounds__(256) swiglu(float* G, const float* U, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
        const float gt = G[i];
        G[i] = gt / (1.0f + __expf(-gt)) * U[i];
    }
}

void run_gemm(const float* A, int lda, const uint16_t* W, int K, float* C, int ldc, int M, int N, int acc,
              hipStream_t s) {
    const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
    hipLaunchKernelGGL(gemm, grid, dim3(256), 0, s, A, lda, W, K, C, ldc, M, N, acc);
}

}  // namespace pf

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
    using namespace pf;
    const int B = a.B, P = a.P, H = a.H, D = a.D, F = a.F, V = a.V;
    const int QD = a.Hq * D, KD = a.Hkv * D, NQKV = QD + 2 * KD;
    auto bf16 = [](const void* p) { return (const uint16_t*)p; };
    // positions [t0, t0 + Pc) of every batch row go through all layers before the next chunk:
    // attention reads the keys and values of earlier chunks from the cache
    for (int t0 = 0; t0 < P; t0 += a.chunk) {
        const int Pc = P - t0 < a.chunk ? P - t0 : a.chunk, M = B * Pc;
        hipLaunchKernelGGL(embed, dim3(M), dim3(256), 0, s, a.tokens, P, t0, Pc, H, V, a.embed, a.X, a.bad, a.err);
        for (int l = 0; l < a.L; ++l) {
            hipLaunchKernelGGL(rmsnorm, dim3(M), dim3(256), 0, s, a.X, (size_t)H, H, bf16(a.attn_norm[l]), a.eps, a.A,
                               (size_t)H);
            run_gemm(a.A, H, bf16(a.wq[l]), H, a.QKV, NQKV, M, QD, 0, s);
            run_gemm(a.A, H, bf16(a.wk[l]), H, a.QKV + QD, NQKV, M, KD, 0, s);
            run_gemm(a.A, H, bf16(a.wv[l]), H, a.QKV + QD + KD, NQKV, M, KD, 0, s);
            hipLaunchKernelGGL(rope_kv, dim3(M), dim3(256), 0, s, a.QKV, NQKV, B, t0, Pc, a.Hq, a.Hkv, D, a.rope, a.kv,
                               l, a.max_seq);
            const unsigned nat = (unsigned)(((size_t)M * a.Hq + 3) / 4);
            if (D == 64)
                hipLaunchKernelGGL(attention<64>, dim3(nat), dim3(256), 0, s, a.QKV, NQKV, a.kv, B, t0, Pc, a.Hq, a.Hkv,
                                   l, a.max_seq, a.O, QD);
            else
                hipLaunchKernelGGL(attention<128>, dim3(nat), dim3(256), 0, s, a.QKV, NQKV, a.kv, B, t0, Pc, a.Hq,
                                   a.Hkv, l, a.max_seq, a.O, QD);
            run_gemm(a.O, QD, bf16(a.wo[l]), QD, a.X, H, M, H, 1, s);  // h += W_o attn
            hipLaunchKernelGGL(rmsnorm, dim3(M), dim3(256), 0, s, a.X, (size_t)H, H, bf16(a.mlp_norm[l]), a.eps, a.A,
                               (size_t)H);
            run_gemm(a.A, H, bf16(a.w_gate[l]), H, a.G, F, M, F, 0, s);
            run_gemm(a.A, H, bf16(a.w_up[l]), H, a.U, F, M, F, 0, s);
            const size_t n = (size_t)M * F;
            hipLaunchKernelGGL(swiglu, dim3((unsigned)std::min<size_t>((n + 255) / 256, 65536)), dim3(256), 0, s, a.G,
                               a.U, n);
            run_gemm(a.G, F, bf16(a.w_down[l]), F, a.X, H, M, H, 1, s);  // h += W_down a
        }
        if (t0 + Pc == P) {
            // the last position of each row: final RMSNorm, then the LM head
            hipLaunchKernelGGL(rmsnorm, dim3(B), dim3(256), 0, s, a.X + (size_t)(Pc - 1) * H, (size_t)Pc * H, H,
                               a.final_norm, a.eps, a.A, (size_t)H);
            run_gemm(a.A, H, a.lm_head, H, a.logits, V, B, V, 0, s);
        }
    }
    return hipGetLastError();
}

// The static scratch of mk_prefill_static: one array per device, for the life
// of the process.  Its device address comes from the runtime (the array's name
// is only a host-side stand-in), looked up once per device with that device
// current.
static __device__ __align__(256) uint8_t scratch[PREFILL_SCRATCH_BYTES];

hipError_t prefill_scratch_address(int device, void** out) {
    constexpr int MAX_DEVICES = 64;
    static std::mutex mu;
    static void* addr[MAX_DEVICES] = {};
    if (device < 0 || device >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[device]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[device] = p;
    }
    *out = addr[device];
    return hipSuccess;
}

}  // namespace mk
