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
// weights, fp32 sums; see gemm).  Causal attention is a tiled online-softmax
// kernel on the same matrix cores; RMSNorm, RoPE + cache append and SwiGLU are
// small vector kernels between them; all on the caller's stream.
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

// Causal attention of every query of the chunk (row m, head h at position t) over cache slots
// 0 .. t of its KV group (earlier chunks' slots were written by their passes), in the tiled
// online-softmax form on the bf16 matrix cores:
//   O[m][h D + d] = sum_j softmax_j(q . k_j / sqrt(D)) v_j[d].
// A block takes 64 queries of one head (a wave per 16) and walks the keys in tiles of 32,
// staged in LDS (K as rows, V transposed).  Per tile a wave computes S^T = K Q^T (q in two
// bf16 terms, K exact in bf16: lane l ends with keys 4 (l/16) + i and 16 + 4 (l/16) + i of
// query l % 16), updates the running max and sum of its query, and adds V^T P^T to O^T with
// those eight probabilities (two bf16 terms) as the B operand: the contraction's key order is
// permuted the same way in both operands, which leaves the sum unchanged.  The products are
// exact and every sum is fp32, as in the per-position form.
typedef float f32x8 __attribute__((ext_vector_type(8)));
template <int D>
__global__ void __launch_bounds__(256) attention(const float* QKV, int ld, const uint16_t* kv, int B, int t0, int Pc,
                                                 int Hq, int Hkv, int layer, int max_seq, float* O, int ldo) {
    constexpr int KT = 32, KS = D / 32, DT = D / 16, LDKS = D + 8, LDV = KT + 8;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * LDKS];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * LDV];
    const int head = blockIdx.y, b = blockIdx.z, g = head / (Hq / Hkv);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lq = lane & 15, lg = lane >> 4;
    const int qb0 = blockIdx.x * 64;             // the block's first query (row of the chunk)
    const int qi = qb0 + wave * 16 + lq;         // this lane's query
    const bool qvalid = qi < Pc;
    const int qr = qvalid ? qi : Pc - 1;         // rows past the chunk repeat its last (not written)
    const int t = t0 + qr;                       // its position
    const int t_blk = t0 + min(qb0 + 63, Pc - 1), t_wave = t0 + min(qb0 + wave * 16 + 15, Pc - 1);
    // q of this lane's query, dims ks * 32 + 8 (l / 16) + j: the B operand of S^T = K Q^T
    const float* qrow = QKV + (size_t)(b * Pc + qr) * ld + (size_t)head * D;
    bf16x8 qh[KS], ql[KS];
    for (int ks = 0; ks < KS; ++ks) {
        const float4 u = *(const float4*)(qrow + ks * 32 + 8 * lg), w = *(const float4*)(qrow + ks * 32 + 8 * lg + 4);
        const f32x8 x = {u.x, u.y, u.z, u.w, w.x, w.y, w.z, w.w};
        qh[ks] = __builtin_convertvector(x, bf16x8);
        ql[ks] = __builtin_convertvector(x - __builtin_convertvector(qh[ks], f32x8), bf16x8);
    }
    const uint16_t* Kb = kv + ((((size_t)layer * 2 + 0) * B + b) * Hkv + g) * (size_t)max_seq * D;
    const uint16_t* Vb = kv + ((((size_t)layer * 2 + 1) * B + b) * Hkv + g) * (size_t)max_seq * D;
    const float scale = rsqrtf((float)D), ninf = -__builtin_inff();
    f32x4 o[DT];
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = ninf, lsum = 0.f;
    for (int j0 = 0; j0 <= t_blk; j0 += KT) {
        __syncthreads();  // every wave is done with the previous tile
        for (int e = threadIdx.x; e < KT * D / 8; e += 256) {
            const int r = e / (D / 8), c = (e % (D / 8)) * 8, j = j0 + r;
            uint4 kk = make_uint4(0u, 0u, 0u, 0u), vv = make_uint4(0u, 0u, 0u, 0u);
            if (j <= t_blk) {
                kk = *(const uint4*)(Kb + (size_t)j * D + c);
                vv = *(const uint4*)(Vb + (size_t)j * D + c);
            }
            *(uint4*)&Ks[r * LDKS + c] = kk;
            const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
            for (int k = 0; k < 4; ++k) {
                Vt[(c + 2 * k) * LDV + r] = (uint16_t)(vw[k] & 0xffffu);
                Vt[(c + 2 * k + 1) * LDV + r] = (uint16_t)(vw[k] >> 16);
            }
        }
        __syncthreads();
        if (j0 > t_wave) continue;  // every query of this wave precedes the tile
        f32x4 st[2];
        for (int kt = 0; kt < 2; ++kt) {
            st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a = *(const bf16x8*)&Ks[(kt * 16 + lq) * LDKS + ks * 32 + 8 * lg];
                st[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh[ks], st[kt], 0, 0, 0);
                st[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[ks], st[kt], 0, 0, 0);
            }
        }
        // lane l: query l % 16, keys j0 + kt 16 + 4 (l / 16) + i
        float sc[8], mx = m;
        for (int kt = 0; kt < 2; ++kt)
            for (int i = 0; i < 4; ++i) {
                const int j = j0 + kt * 16 + 4 * lg + i;
                const float v = j <= t ? st[kt][i] * scale : ninf;
                sc[kt * 4 + i] = v;
                mx = fmaxf(mx, v);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));  // finite: key 0 of the first tile precedes every query
        const float corr = __expf(m - mx);
        float ps = 0.f;
        f32x8 pv;
        for (int k = 0; k < 8; ++k) {
            pv[k] = __expf(sc[k] - mx);
            ps += pv[k];
        }
        ps += __shfl_xor(ps, 16);
        ps += __shfl_xor(ps, 32);
        lsum = lsum * corr + ps;
        m = mx;
        const bf16x8 ph = __builtin_convertvector(pv, bf16x8);
        const bf16x8 pl = __builtin_convertvector(pv - __builtin_convertvector(ph, f32x8), bf16x8);
        for (int dt = 0; dt < DT; ++dt) {
            o[dt] *= corr;
            // V^T rows dt 16 + l % 16, keys 4 (l / 16) .. +3 and 16 + 4 (l / 16) .. +3
            const uint16_t* vr = &Vt[(dt * 16 + lq) * LDV];
            const uint2 v0 = *(const uint2*)(vr + 4 * lg), v1 = *(const uint2*)(vr + 16 + 4 * lg);
            const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ph, o[dt], 0, 0, 0);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pl, o[dt], 0, 0, 0);
        }
    }
    // lane l holds O^T[dt 16 + 4 (l / 16) + i][query l % 16]
    if (qvalid) {
        const float inv = 1.0f / lsum;
        float* out = O + (size_t)(b * Pc + qi) * ldo + (size_t)head * D;
        for (int dt = 0; dt < DT; ++dt)
            for (int i = 0; i < 4; ++i) out[dt * 16 + 4 * lg + i] = o[dt][i] * inv;
    }
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
            const dim3 agrid((unsigned)((Pc + 63) / 64), (unsigned)a.Hq, (unsigned)B);
            if (D == 64)
                hipLaunchKernelGGL(attention<64>, agrid, dim3(256), 0, s, a.QKV, NQKV, a.kv, B, t0, Pc, a.Hq, a.Hkv, l,
                                   a.max_seq, a.O, QD);
            else
                hipLaunchKernelGGL(attention<128>, agrid, dim3(256), 0, s, a.QKV, NQKV, a.kv, B, t0, Pc, a.Hq, a.Hkv,
                                   l, a.max_seq, a.O, QD);
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
