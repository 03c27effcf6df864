// gdn_prefill.hip -- chunked prefill of a prompt (repository "Architecture"
// page: the prompt is prefilled before the decode loop; CPU page, exactness
// section: the chunked form and the token-by-token form are the same algebra
// and differ only in rounding).
//
// Per value head and chunk of n <= 64 tokens starting from state S0, with
// G_t the inclusive cumulative log-decay inside the chunk (G_t = sum log
// alpha), the recurrence folds into (derivation: the chunk-form test)
//   A    = strict-lower( beta_i e^{G_i - G_j} k_i.k_j ),   T = (I + A)^-1
//   U    = T (beta (.) V) - T (beta e^G (.) K) S0^T  =  U~ - W~ S0^T
//   O    = s ( e^G (.) Q S0^T + P U ),   P = lower-incl( e^{G_i - G_j} q_i.k_j )
//   S_n  = e^{G_n} S0 + U^T (e^{G_n - G} (.) K)
// Only differences G_i - G_j with i >= j are exponentiated, so nothing
// overflows however strong the decay.
//
// Work split for MI355X, per segment of at most 2,048 tokens:
//   conv  (parallel over 16-token blocks x q/k heads): conv + SiLU of the
//         q/k head's channels and of its value heads' channels, q/k L2 norm;
//         writes fp16 q^, k^, k^ transposed per chunk and v transposed per
//         chunk.  Small LDS, many waves per CU.
//   tri   (parallel over value heads x chunks): gates and G, K K^T and Q K^T
//         on MFMA, A, the blocked inverse T in fp32 (16x16 diagonal blocks by
//         substitution, off-diagonal blocks by block products), then
//         U~ = T (beta V) and W~ = T (beta e^G K) on MFMA, and P.
//   scan  (sequential over chunks; one workgroup per (sequence, value head,
//         32-row slice of the state), one workgroup per CU): Z = W~ S0^T and
//         Y = Q S0^T, U = U~ - Z, O = s (e^G Y + P U),
//         S <- e^{G_n} S + U^T (e^{G_n - G} K), all on 16x16x32 fp16 MFMAs,
//         two barriers per chunk.  Four waves carry the state (fp32, in
//         registers across chunks); four more compute and store o off the
//         state's critical path.  Operands stream through a four-stage
//         register ring, three chunks ahead.  Workgroups of one q/k head sit
//         on one XCD and share its L2.
// The workspace holds one segment (about 114 MB at the 27B-class shape),
// whatever the prompt length, small enough to live in the Infinity Cache.
#include <algorithm>
#include <utility>

#include "gdn_core.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace pf {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;       // head width handled by the prefill kernels
constexpr int CH = 64;       // chunk length
constexpr int SEG = 2048;    // tokens per segment
constexpr int TB = 16;       // tokens per conv workgroup
constexpr int DS = 32;       // state rows per scan workgroup
constexpr int NS = D / DS;   // scan workgroups per value head
constexpr int MP = CH + 1;   // fp32 pitch of a 64x64 matrix row in LDS
constexpr int HP = CH + 8;   // fp16 pitch of a 64-token row in LDS
constexpr float kScale = Scale<D>::value;

// Workspace of one segment; SP = token pitch (segment length rounded to 64),
// NC = SP / 64 chunks.  Every chunk operand is stored in the order the MFMA
// fragments read it (a_off / b_off / c_off below), so that each wave's
// operand load is one contiguous run of 64 lanes x 16 bytes:
//   q, k  fp16 [B][Hk][NC][64 x 128 A order]   normalised q^, k^ (zero past the prompt)
//   kt    fp16 [B][Hk][NC][64 x 128 B order]   k^ with the token index as k
//   vt    fp16 [B][Hv][NC][64 x 128 B order]   v with the token index as k
//   ut    fp16 [B][Hv][NC][64 x 128 C order]   U~ = T (beta V)
//   wt    fp16 [B][Hv][NC][64 x 128 A order]   W~ = T (beta e^G K)
//   P     fp16 [B][Hv][NC][64 x 64 A order]
//   eg    f32  [B][Hv][SP]                     e^{G_t}
//   egd   f32  [B][Hv][SP]                     e^{G_last - G_t}
struct Ws {
    _Float16 *q, *k, *kt, *vt, *ut, *wt, *P;
    float *eg, *egd;
};

inline size_t seg_pitch(int T) { return static_cast<size_t>(T >= SEG ? SEG : (T + CH - 1) / CH * CH); }

inline size_t ws_bytes(int B, int Hk, int Hv, size_t SP) {
    const size_t per_tok = 3ull * Hk * D * 2 + 3ull * Hv * D * 2 + Hv * CH * 2ull + Hv * 8ull;
    return static_cast<size_t>(B) * SP * per_tok + 256 * 10;
}

inline Ws carve(void* base, int B, int Hk, int Hv, size_t SP) {
    auto align = [](uintptr_t p) { return (p + 255) & ~static_cast<uintptr_t>(255); };
    uintptr_t p = align(reinterpret_cast<uintptr_t>(base));
    const size_t nk = static_cast<size_t>(B) * Hk * SP * D, nv = static_cast<size_t>(B) * Hv * SP * D;
    const size_t nm = static_cast<size_t>(B) * Hv * SP * CH, ng = static_cast<size_t>(B) * Hv * SP;
    Ws w;
    auto take16 = [&](size_t n) { _Float16* r = reinterpret_cast<_Float16*>(p); p = align(p + n * 2); return r; };
    auto take32 = [&](size_t n) { float* r = reinterpret_cast<float*>(p); p = align(p + n * 4); return r; };
    w.q = take16(nk);
    w.k = take16(nk);
    w.kt = take16(nk);
    w.vt = take16(nv);
    w.ut = take16(nv);
    w.wt = take16(nv);
    w.P = take16(nm);
    w.eg = take32(ng);
    w.egd = take32(ng);
    return w;
}

__device__ __forceinline__ f4 mma(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
__device__ __forceinline__ h8 ld8(const _Float16* p) { return *reinterpret_cast<const h8*>(p); }
__device__ __forceinline__ f4 zero4() { return f4{0.0f, 0.0f, 0.0f, 0.0f}; }

// Fragment orders of one chunk's matrices for 16x16x32 MFMAs.  A fragment
// (16 rows x 32 k): lane (lq, lr) holds row lr, k 8 lq .. 8 lq + 7.  B fragment
// (32 k x 16 columns): lane (lq, lr) holds column lr, k 8 lq .. 8 lq + 7.  C
// tile (16 x 16): lane (lq, lr) holds rows 4 lq .. 4 lq + 3 of column lr.
// Tiles are laid out one after another, 64 lanes x 8 (A, B) or x 4 (C) fp16.
//   a_off: M[row][k], ks k-steps per row tile;  b_off: M[k][col], ks k-steps
//   per column tile;  c_off: M[row][col], nct column tiles per row tile.
__device__ __forceinline__ int a_off(int row, int k, int ks) {
    return (((row >> 4) * ks + (k >> 5)) * 64 + ((k & 31) >> 3) * 16 + (row & 15)) * 8 + (k & 7);
}
__device__ __forceinline__ int b_off(int k, int col, int ks) {
    return (((col >> 4) * ks + (k >> 5)) * 64 + ((k & 31) >> 3) * 16 + (col & 15)) * 8 + (k & 7);
}
__device__ __forceinline__ int c_off(int row, int col, int nct) {
    return (((row >> 4) * nct + (col >> 4)) * 64 + ((row & 15) >> 2) * 16 + (col & 15)) * 4 + (row & 3);
}
// One A or B fragment of tile `tile` in a fragment-ordered matrix.
__device__ __forceinline__ h8 ldfrag(const _Float16* m, int tile, int lane) { return ld8(m + tile * 512 + lane * 8); }
constexpr int kChunkQK = CH * D;   // fp16 elements of one chunk of q, k, k^T, v^T, U~, W~
constexpr int kChunkP = CH * CH;   // fp16 elements of one chunk of P

// Prefill stores q^, k^ and v as fp16 (relative step 2^-11), so its conv and
// norm use the hardware exp2, reciprocal and reciprocal square root (about one
// ulp of fp32 each) instead of the correctly rounded library calls the
// token-by-token path shares.
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float conv_silu_fast(const float w[4], const float win[4]) {
    float acc = w[0] * win[0];
    acc = __builtin_fmaf(w[1], win[1], acc);
    acc = __builtin_fmaf(w[2], win[2], acc);
    acc = __builtin_fmaf(w[3], win[3], acc);
    return acc * __builtin_amdgcn_rcpf(1.0f + fast_exp(-acc));
}

// ------------------------------------------------------------ conv + norm

template <typename Act>
__global__ __launch_bounds__(640) void conv_kernel(const Act* __restrict__ x, const Act* __restrict__ tail,
                                                   const Act* __restrict__ w, Ws ws, int T, int seg0, int SP,
                                                   int nblk, int B, int Hk, int Hv, int C) {
    __shared__ float ys[TB][2 * D];                  // q~ | k~ of the block, fp32
    __shared__ __align__(16) _Float16 qkh[2][TB][D]; // q^, k^ of the block, fp16
    // The CH / TB blocks of one chunk write disjoint pieces of the same
    // 128-byte lines of v^T and k^T.  They share an XCD (blockIdx % 8 picks
    // it), so the pieces merge in one L2 instead of reaching memory as
    // partial lines.
    constexpr int BPC = CH / TB;                     // blocks per chunk
    const int nch = nblk / BPC;
    const int xcd = blockIdx.x % 8, r8 = blockIdx.x / 8;
    const int chunk_id = (r8 / BPC) * 8 + xcd;       // (sequence, q/k head, chunk of the segment)
    if (chunk_id >= B * Hk * nch)
        return;
    const int tb = (chunk_id % nch) * BPC + r8 % BPC;
    const int g = (chunk_id / nch) % Hk;
    const int bq = chunk_id / (nch * Hk);
    const int G = Hv / Hk;
    const int NC = SP / CH;
    const int t0 = seg0 + tb * TB;                   // prompt index of the block's first token
    const int sl = tb * TB;                          // segment index of the same token
    const int cl = sl / CH, co = sl % CH;            // its chunk and offset in the chunk
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const Act* xb = x + static_cast<size_t>(bq) * T * C;
    const Act* tbq = tail + static_cast<size_t>(bq) * C * 4;
    const int per_group = (2 + G) * D;

    // Two channels per thread (the block has per_group / 2 threads); the
    // window loads of both are issued before either is used.
    int chs[2], cs[2];
    float wfs[2][4];
    float hist[2][TB + 3];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int ch0 = threadIdx.x + k * blockDim.x;
        const int ch = ch0 < per_group ? ch0 : per_group - 1;
        chs[k] = ch0;
        cs[k] = ch < D ? g * D + ch : ch < 2 * D ? Hk * D + g * D + (ch - D) : 2 * Hk * D + G * g * D + (ch - 2 * D);
        Quad<Act>::to_float(Quad<Act>::load(w + static_cast<size_t>(cs[k]) * 4), wfs[k]);
        // unconditional loads from selected addresses: all of them in flight at once
#pragma unroll
        for (int m = 0; m < TB + 3; ++m) {
            const int t = t0 + m - 3;
            const int tc = t < T ? t : T - 1;
            const Act* src = t < 0 ? tbq + static_cast<size_t>(cs[k]) * 4 + 4 + t : xb + static_cast<size_t>(tc) * C + cs[k];
            hist[k][m] = widen(*src);
        }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int ch = chs[k];
        if (ch >= per_group)
            continue;
        float yv[TB];
#pragma unroll
        for (int j = 0; j < TB; ++j)
            yv[j] = (t0 + j < T) ? conv_silu_fast(wfs[k], &hist[k][j]) : 0.0f;
        if (ch < 2 * D) {
#pragma unroll
            for (int j = 0; j < TB; ++j)
                ys[j][ch] = yv[j];
        } else {
            const int h = G * g + (ch - 2 * D) / D;
            const int d = (ch - 2 * D) % D;
            h8 lo, hi;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                lo[j] = static_cast<_Float16>(yv[j]);
                hi[j] = static_cast<_Float16>(yv[8 + j]);
            }
            // tokens co .. co + 15 of column d: two B-order runs of 8
            _Float16* vc = ws.vt + ((static_cast<size_t>(bq) * Hv + h) * NC + cl) * kChunkQK;
            *reinterpret_cast<h8*>(vc + b_off(co, d, CH / 32)) = lo;
            *reinterpret_cast<h8*>(vc + b_off(co + 8, d, CH / 32)) = hi;
        }
    }
    __syncthreads();
    const int nwaves = blockDim.x / kWave;
    for (int vec = wave; vec < 2 * TB; vec += nwaves) {
        const int tl = vec >> 1, which = vec & 1;
        const float e0 = ys[tl][which * D + lane];
        const float e1 = ys[tl][which * D + lane + kWave];
        const float ss = group_sum<kWave>(__builtin_fmaf(e1, e1, e0 * e0));
        const float r = __builtin_amdgcn_rsqf(ss + kEps);
        qkh[which][tl][lane] = static_cast<_Float16>(e0 * r);
        qkh[which][tl][lane + kWave] = static_cast<_Float16>(e1 * r);
    }
    __syncthreads();
    // The block is row tile co / 16 of the chunk: q^ and k^ in A order (16
    // tokens x 8 keys per run), k^ in B order (8 tokens x 1 key per run).
    const size_t qkc = ((static_cast<size_t>(bq) * Hk + g) * NC + cl) * kChunkQK;
    for (int idx = threadIdx.x; idx < 2 * TB * D / 8; idx += blockDim.x) {
        const int which = idx / (TB * D / 8), f = idx % (TB * D / 8);
        const int tl = f % TB, k0 = 8 * (f / TB);
        const h8 v = *reinterpret_cast<const h8*>(&qkh[which][tl][k0]);
        *reinterpret_cast<h8*>((which ? ws.k : ws.q) + qkc + a_off(co + tl, k0, D / 32)) = v;
    }
    for (int idx = threadIdx.x; idx < TB / 8 * D; idx += blockDim.x) {
        const int d = idx % D, half = idx / D;
        h8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            v[j] = qkh[1][8 * half + j][d];
        *reinterpret_cast<h8*>(ws.kt + qkc + b_off(co + 8 * half, d, CH / 32)) = v;
    }
}

// ------------------------------------------------------------ tri

struct alignas(16) TriSmem {
    float A[CH][MP];              // after the inverse: W~ staged as fp16 [64][128]
    float T[CH][MP];
    _Float16 Ps[CH][CH + 8];      // P staged for its A-order store
    float tmp[3][16][17];
    float G[CH];     // cumulative log2 decay inside the chunk
    float beta[CH];
    float bv[CH];    // beta_t            (scales V in U~)
    float bk[CH];    // beta_t e^{G_t}    (scales K in W~)
};

__global__ __launch_bounds__(256) void tri_kernel(const float* __restrict__ a, const float* __restrict__ bg, Ws ws,
                                                  int T, int seg0, int SP, int nch, int Hk, int Hv) {
    __shared__ TriSmem sm;
    const int cl = blockIdx.x % nch;
    const int h = (blockIdx.x / nch) % Hv;
    const int bq = blockIdx.x / (nch * Hv);
    const int g = h / (Hv / Hk);
    const int NC = SP / CH;
    const int t_base = seg0 + cl * CH;
    const int n = min(CH, T - t_base);
    const int s0 = cl * CH;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int lr = lane & 15, lq = lane >> 4;
    const size_t hs = (static_cast<size_t>(bq) * Hv + h) * SP + s0;   // this head's token row base

    // Gate inputs first, then every operand fragment this wave needs, so that
    // waiting for the gates does not wait for the fragments.
    float av = 0.0f, bv = 0.0f;
    if (wave == 0 && lane < n) {
        const size_t idx = (static_cast<size_t>(bq) * T + t_base + lane) * Hv + h;
        av = a[idx];
        bv = bg[idx];
    }
    // Every operand fragment this wave needs is requested up front.
    //   K K^T / Q K^T: wave w computes row block w (tiles (w, J), J <= w).
    //   U~ / W~: wave w computes column tiles 2w and 2w+1 for all token rows.
    const size_t qkc = ((static_cast<size_t>(bq) * Hk + g) * NC + cl) * kChunkQK;
    const size_t hc = ((static_cast<size_t>(bq) * Hv + h) * NC + cl) * kChunkQK;
    const _Float16* qg = ws.q + qkc;
    const _Float16* kg = ws.k + qkc;
    const _Float16* vth = ws.vt + hc;
    const _Float16* ktg = ws.kt + qkc;
    h8 qa[4], ka[4], kb[3][4], vb[2][2], kt[2][2];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        qa[s] = ldfrag(qg, 4 * wave + s, lane);
        ka[s] = ldfrag(kg, 4 * wave + s, lane);
#pragma unroll
        for (int J = 0; J < 3; ++J)
            kb[J][s] = ldfrag(kg, 4 * (J < wave ? J : wave) + s, lane);
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            vb[tt][s] = ldfrag(vth, 2 * (2 * wave + tt) + s, lane);
            kt[tt][s] = ldfrag(ktg, 2 * (2 * wave + tt) + s, lane);
        }

    if (wave == 0) {
        float la = 0.0f, be = 0.0f;
        if (lane < n) {
            la = -(fmaxf(av, 0.0f) + log1pf(expf(-fabsf(av))));
            be = 1.0f / (1.0f + expf(-bv));
        }
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const float up = __shfl_up(la, off, kWave);
            if (lane >= off)
                la += up;
        }
        const float l2 = la * kLog2e;             // G in log2 units
        const float glast = __shfl(l2, kWave - 1, kWave);
        const float eg = __builtin_amdgcn_exp2f(l2);
        sm.G[lane] = l2;
        sm.beta[lane] = be;
        sm.bv[lane] = be;
        sm.bk[lane] = be * eg;
        ws.eg[hs + lane] = eg;
        ws.egd[hs + lane] = __builtin_amdgcn_exp2f(glast - l2);
    }
    __syncthreads();

    // K K^T -> A and Q K^T -> P for row block w; the blocks right of the
    // diagonal are zero in P and in T.
#pragma unroll
    for (int J = 0; J < 4; ++J) {
        const int i0 = 16 * wave + 4 * lq, j = 16 * J + lr;
        if (J <= wave) {
            f4 kk = zero4(), qk = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const h8 b = (J == wave) ? ka[s] : kb[J < 3 ? J : 0][s];
                kk = mma(ka[s], b, kk);
                qk = mma(qa[s], b, qk);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = i0 + r;
                const float dg = (i >= j) ? __builtin_amdgcn_exp2f(sm.G[i] - sm.G[j]) : 0.0f;
                sm.Ps[i][j] = static_cast<_Float16>(dg * qk[r]);
                sm.A[i][j] = (i > j) ? sm.beta[i] * dg * kk[r] : 0.0f;
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sm.Ps[i0 + r][j] = static_cast<_Float16>(0.0f);
                sm.T[i0 + r][j] = 0.0f;
            }
        }
    }
    __syncthreads();
    {
        _Float16* Pc = ws.P + ((static_cast<size_t>(bq) * Hv + h) * NC + cl) * kChunkP;
        for (int idx = threadIdx.x; idx < kChunkP / 8; idx += blockDim.x) {
            const int i = idx % CH, j0 = 8 * (idx / CH);
            *reinterpret_cast<h8*>(Pc + a_off(i, j0, CH / 32)) = *reinterpret_cast<const h8*>(&sm.Ps[i][j0]);
        }
    }

    // diagonal 16x16 blocks of (I + A)^-1: wave 0, lane = (block, column)
    if (wave == 0) {
        const int o = 16 * lq, j = lr;
        float X[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = (i == j) ? 1.0f : 0.0f;
#pragma unroll
            for (int k = 0; k < i; ++k)
                s = __builtin_fmaf(-sm.A[o + i][o + k], X[k], s);
            X[i] = s;
            sm.T[o + i][o + j] = s;
        }
    }
    __syncthreads();
    // off-diagonal blocks, one block diagonal at a time: T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ
    for (int lvl = 1; lvl < 4; ++lvl) {
        const int nb = 4 - lvl;
        for (int e = threadIdx.x; e < nb * 256; e += blockDim.x) {
            const int q = e / 256, r = (e / 16) % 16, c = e % 16;
            const int I = lvl + q, J = q;
            float s = 0.0f;
            for (int K = J; K < I; ++K)
#pragma unroll
                for (int k = 0; k < 16; ++k)
                    s = __builtin_fmaf(sm.A[16 * I + r][16 * K + k], sm.T[16 * K + k][16 * J + c], s);
            sm.tmp[q][r][c] = s;
        }
        __syncthreads();
        for (int e = threadIdx.x; e < nb * 256; e += blockDim.x) {
            const int q = e / 256, r = (e / 16) % 16, c = e % 16;
            const int I = lvl + q, J = q;
            float s = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; ++k)
                s = __builtin_fmaf(sm.T[16 * I + r][16 * I + k], sm.tmp[q][k][c], s);
            sm.T[16 * I + r][16 * J + c] = -s;
        }
        __syncthreads();
    }

    // U~ = T (beta V) and W~ = T (beta e^G K): wave w owns column tiles 2w, 2w+1
    h8 vsc[2][2], ksc[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        float fv[8], fk[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            fv[e] = sm.bv[32 * s + 8 * lq + e];
            fk[e] = sm.bk[32 * s + 8 * lq + e];
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                vsc[tt][s][e] = static_cast<_Float16>(static_cast<float>(vb[tt][s][e]) * fv[e]);
                ksc[tt][s][e] = static_cast<_Float16>(static_cast<float>(kt[tt][s][e]) * fk[e]);
            }
    }
    _Float16* uto = ws.ut + hc;
    _Float16* wst = reinterpret_cast<_Float16*>(&sm.A[0][0]);   // W~ staging [64][128] (A is no longer needed)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        h8 tf[2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                tf[s][e] = static_cast<_Float16>(sm.T[16 * m + lr][32 * s + 8 * lq + e]);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            f4 u = zero4(), wv = zero4();
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                u = mma(tf[s], vsc[tt][s], u);
                wv = mma(tf[s], ksc[tt][s], wv);
            }
            const int d = 16 * (2 * wave + tt) + lr;
            typedef _Float16 h4 __attribute__((ext_vector_type(4)));
            h4 uh;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uh[r] = static_cast<_Float16>(u[r]);
                wst[(16 * m + 4 * lq + r) * D + d] = static_cast<_Float16>(wv[r]);
            }
            *reinterpret_cast<h4*>(uto + c_off(16 * m + 4 * lq, d, D / 16)) = uh;
        }
    }
    __syncthreads();
    _Float16* wto = ws.wt + hc;
    for (int idx = threadIdx.x; idx < kChunkQK / 8; idx += blockDim.x) {
        const int t = idx % CH, k0 = 8 * (idx / CH);
        *reinterpret_cast<h8*>(wto + a_off(t, k0, D / 32)) = *reinterpret_cast<const h8*>(&wst[t * D + k0]);
    }
}

// ------------------------------------------------------------ scan

// The scan workgroup owns DS rows of one value head's state and has two roles
// of four waves.  State waves carry the recurrence: Z = W~ S0^T, U = U~ - Z,
// S <- e^{G_n} S + U^T (e^{G_n - G} K), the state in fp32 registers across
// chunks.  Output waves compute Y = Q S0^T and P U and store o.  The roles meet
// at two barriers per chunk; S0 and U^T pass through LDS, double-buffered by
// chunk parity.
//
// The workgroup's operands of a chunk (W~, K^T, Q and P of its head; U~ of its
// rows) are read once per workgroup, so the chip-wide operand traffic is
// (value heads x 128 / DS) copies per chunk: DS = 32 keeps it within what the
// L2 delivers while one workgroup per CU keeps every state slice resident.
// Each wave streams its operands through a ring of kScanRing register stages,
// so the chunk it computes was requested kScanRing - 1 chunks earlier.  The
// chunk loop body holds kScanRing chunks, which keeps every ring slot in fixed
// registers while the code stays small enough for the instruction cache.
constexpr int kScanRing = 4;

struct alignas(16) ScanSmem {
    _Float16 s0[2][DS][D + 8];   // S0 slice, fp16, [row][key]
    _Float16 ut[2][DS][HP];      // U^T [row][t]
    _Float16 utd[DS][HP];        // U^T scaled by e^{G_last - G} (state waves only)
};

struct StateOps {
    h8 wf[4], kf[2][2];
    uint2 u[DS / 16];   // four fp16 U~ values per row tile
    f4 egd;
    float eglast;
};

struct OutOps {
    h8 qf[4], pf[2];
    f4 eg;
};

struct ScanCtx {
    size_t gbase, hbase, pbase, ktbase, utbase;
    int w, lr, lq, row0;   // w: this wave's index within its role
};

__device__ __forceinline__ void load_state(StateOps& op, const Ws& ws, const ScanCtx& c, int cl) {
    const int s0 = cl * CH;
    const int lane = 16 * c.lq + c.lr;
    const _Float16* wc = ws.wt + (c.utbase + cl) * kChunkQK;
    const _Float16* kc = ws.kt + (c.ktbase + cl) * kChunkQK;
    const _Float16* uc = ws.ut + (c.utbase + cl) * kChunkQK;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        op.wf[s] = ldfrag(wc, 4 * c.w + s, lane);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
            op.kf[tt][s] = ldfrag(kc, 2 * (2 * c.w + tt) + s, lane);
#pragma unroll
    for (int it = 0; it < DS / 16; ++it)
        op.u[it] = *reinterpret_cast<const uint2*>(uc + ((c.w * (D / 16) + c.row0 / 16 + it) * 64 + lane) * 4);
    op.egd = *reinterpret_cast<const f4*>(ws.egd + c.hbase + s0 + 16 * c.w + 4 * c.lq);
    op.eglast = ws.eg[c.hbase + s0 + CH - 1];
}

__device__ __forceinline__ void load_out(OutOps& op, const Ws& ws, const ScanCtx& c, int cl) {
    const int s0 = cl * CH;
    const int lane = 16 * c.lq + c.lr;
    const _Float16* qc = ws.q + (c.ktbase + cl) * kChunkQK;
    const _Float16* pc = ws.P + (c.pbase + cl) * kChunkP;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        op.qf[s] = ldfrag(qc, 4 * c.w + s, lane);
#pragma unroll
    for (int s = 0; s < 2; ++s)
        op.pf[s] = ldfrag(pc, 2 * c.w + s, lane);
    op.eg = *reinterpret_cast<const f4*>(ws.eg + c.hbase + s0 + 16 * c.w + 4 * c.lq);
}

// x S0^T for one 16-token tile and the 16 state rows starting at s0, keys
// split into two independent chains.
__device__ __forceinline__ f4 times_s0(const h8 (&a)[4], const _Float16 (*s0)[D + 8], int lr, int lq) {
    f4 z0 = zero4(), z1 = zero4();
    z0 = mma(a[0], ld8(&s0[lr][8 * lq]), z0);
    z1 = mma(a[2], ld8(&s0[lr][64 + 8 * lq]), z1);
    z0 = mma(a[1], ld8(&s0[lr][32 + 8 * lq]), z0);
    z1 = mma(a[3], ld8(&s0[lr][96 + 8 * lq]), z1);
    return z0 + z1;
}

// sacc[it][tt]: rows 16*it.., keys 16*(2w+tt).. of the slice (C layout: row
// 4*lq + r, column lr).
template <int PAR>
__device__ __forceinline__ void state_chunk(const StateOps& op, ScanSmem& sm, f4 (&sacc)[DS / 16][2],
                                            const ScanCtx& c) {
    const int w = c.w, lr = c.lr, lq = c.lq;
#pragma unroll
    for (int it = 0; it < DS / 16; ++it)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sm.s0[PAR][16 * it + 4 * lq + r][16 * (2 * w + tt) + lr] = static_cast<_Float16>(sacc[it][tt][r]);
    __syncthreads();
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int it = 0; it < DS / 16; ++it) {
        const f4 Z = times_s0(op.wf, &sm.s0[PAR][16 * it], lr, lq);
        const h4 uh = __builtin_bit_cast(h4, op.u[it]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * w + 4 * lq + r;
            const float U = static_cast<float>(uh[r]) - Z[r];
            sm.ut[PAR][16 * it + lr][t] = static_cast<_Float16>(U);
            sm.utd[16 * it + lr][t] = static_cast<_Float16>(U * op.egd[r]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < DS / 16; ++it)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[it][tt][r] *= op.eglast;
#pragma unroll
            for (int s = 0; s < 2; ++s)
                sacc[it][tt] = mma(ld8(&sm.utd[16 * it + lr][32 * s + 8 * lq]), op.kf[tt][s], sacc[it][tt]);
        }
}

// orow points at the chunk's first token row of o for this head and slice; a
// final partial chunk stores only its n valid tokens.
template <int PAR, bool MASKED>
__device__ __forceinline__ void out_chunk(const OutOps& op, ScanSmem& sm, const ScanCtx& c,
                                          float* __restrict__ orow, int n, size_t ostride) {
    const int w = c.w, lr = c.lr, lq = c.lq;
    __syncthreads();
    f4 Y[DS / 16];
#pragma unroll
    for (int it = 0; it < DS / 16; ++it)
        Y[it] = times_s0(op.qf, &sm.s0[PAR][16 * it], lr, lq);
    __syncthreads();
#pragma unroll
    for (int it = 0; it < DS / 16; ++it) {
        f4 PU = zero4();
#pragma unroll
        for (int s = 0; s < 2; ++s)
            PU = mma(op.pf[s], ld8(&sm.ut[PAR][16 * it + lr][32 * s + 8 * lq]), PU);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * w + 4 * lq + r;
            if (!MASKED || t < n)
                orow[static_cast<size_t>(t) * ostride + 16 * it + lr] =
                    kScale * __builtin_fmaf(op.eg[r], Y[it][r], PU[r]);
        }
    }
}

__global__ __launch_bounds__(512, 2) void scan_kernel(float* __restrict__ S, float* __restrict__ o, Ws ws, int T,
                                                      int seg0, int SP, int nch, int B, int Hk, int Hv) {
    __shared__ ScanSmem sm;
    const int G = Hv / Hk;
    // workgroups of one (sequence, q/k head) share an XCD: blockIdx % 8 picks the XCD
    const int xcd = blockIdx.x % 8, r8 = blockIdx.x / 8;
    const int gu = (r8 / (G * NS)) * 8 + xcd;
    if (gu >= B * Hk)
        return;
    const int rem = r8 % (G * NS);
    const int bq = gu / Hk, g = gu % Hk, h = G * g + rem / NS, row0 = (rem % NS) * DS;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const bool state_role = wave < 4;
    const int NC = SP / CH;
    ScanCtx c;
    c.w = wave & 3;
    c.lr = lane & 15;
    c.lq = lane >> 4;
    c.row0 = row0;
    c.gbase = (static_cast<size_t>(bq) * Hk + g) * SP;   // token rows of q/k head g
    c.hbase = (static_cast<size_t>(bq) * Hv + h) * SP;   // token rows of value head h
    c.pbase = (static_cast<size_t>(bq) * Hv + h) * NC;
    c.utbase = c.pbase;
    c.ktbase = (static_cast<size_t>(bq) * Hk + g) * NC;
    const int len = min(SEG, T - seg0);
    const int nfull = len / CH, tailn = len % CH;
    // Chunk nfull (if tailn > 0) is partial: its workspace rows past the
    // prompt are zero, so the state waves treat it like any other.

    if (state_role) {
        float* Sh = S + ((static_cast<size_t>(bq) * Hv + h) * D + row0) * D;
        f4 sacc[DS / 16][2];
#pragma unroll
        for (int it = 0; it < DS / 16; ++it)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sacc[it][tt][r] = Sh[(16 * it + 4 * c.lq + r) * D + 16 * (2 * c.w + tt) + c.lr];
        StateOps ring[kScanRing];
#pragma unroll
        for (int p = 0; p < kScanRing; ++p)
            load_state(ring[p], ws, c, min(p, nch - 1));
        // chunk cl uses ring slot cl % kScanRing and LDS parity cl & 1, both
        // fixed per position in the unrolled body because cl0 % kScanRing == 0
        auto step = [&](auto pc, int cl) {
            constexpr int P = decltype(pc)::value;
            state_chunk<P & 1>(ring[P], sm, sacc, c);
            load_state(ring[P], ws, c, min(cl + kScanRing, nch - 1));
        };
        int cl0 = 0;
        for (; cl0 + kScanRing <= nch; cl0 += kScanRing) {
            step(std::integral_constant<int, 0>{}, cl0);
            step(std::integral_constant<int, 1>{}, cl0 + 1);
            step(std::integral_constant<int, 2>{}, cl0 + 2);
            step(std::integral_constant<int, 3>{}, cl0 + 3);
        }
        if (cl0 < nch)
            step(std::integral_constant<int, 0>{}, cl0);
        if (cl0 + 1 < nch)
            step(std::integral_constant<int, 1>{}, cl0 + 1);
        if (cl0 + 2 < nch)
            step(std::integral_constant<int, 2>{}, cl0 + 2);
#pragma unroll
        for (int it = 0; it < DS / 16; ++it)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Sh[(16 * it + 4 * c.lq + r) * D + 16 * (2 * c.w + tt) + c.lr] = sacc[it][tt][r];
    } else {
        const size_t ostride = static_cast<size_t>(Hv) * D;
        float* obase = o + ((static_cast<size_t>(bq) * T + seg0) * Hv + h) * D + row0;
        OutOps ring[kScanRing];
#pragma unroll
        for (int p = 0; p < kScanRing; ++p)
            load_out(ring[p], ws, c, min(p, nch - 1));
        auto step = [&](auto pc, int cl) {
            constexpr int P = decltype(pc)::value;
            float* orow = obase + static_cast<size_t>(cl) * CH * ostride;
            if (cl < nfull)
                out_chunk<P & 1, false>(ring[P], sm, c, orow, CH, ostride);
            else
                out_chunk<P & 1, true>(ring[P], sm, c, orow, tailn, ostride);
            load_out(ring[P], ws, c, min(cl + kScanRing, nch - 1));
        };
        int cl0 = 0;
        for (; cl0 + kScanRing <= nch; cl0 += kScanRing) {
            step(std::integral_constant<int, 0>{}, cl0);
            step(std::integral_constant<int, 1>{}, cl0 + 1);
            step(std::integral_constant<int, 2>{}, cl0 + 2);
            step(std::integral_constant<int, 3>{}, cl0 + 3);
        }
        if (cl0 < nch)
            step(std::integral_constant<int, 0>{}, cl0);
        if (cl0 + 1 < nch)
            step(std::integral_constant<int, 1>{}, cl0 + 1);
        if (cl0 + 2 < nch)
            step(std::integral_constant<int, 2>{}, cl0 + 2);
    }
}

// New tail = the last four raw inputs of (old tail ++ the prompt).
template <typename Act>
__global__ __launch_bounds__(256) void tail_kernel(const Act* __restrict__ x, Act* __restrict__ tail, int T, int C,
                                                   int64_t total) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= total)
        return;
    const int c = static_cast<int>(i % C);
    const int64_t b = i / C;
    using Q = Quad<Act>;
    typename Q::raw t = Q::load(tail + i * 4);
    const int first = T > 4 ? T - 4 : 0;
    for (int s = first; s < T; ++s)
        t = Q::push(t, x[(b * T + s) * C + c]);
    Q::store(tail + i * 4, t);
}

}  // namespace pf

size_t prefill_workspace_bytes(const Geo& g, int T) {
    if (g.D != pf::D || g.Hv / g.Hk > 8)
        return 0;
    return pf::ws_bytes(g.B, g.Hk, g.Hv, pf::seg_pitch(T));
}

hipError_t launch_prefill(const Geo& g, float* S, void* tail, const void* w, int T, const void* x, const float* a,
                          const float* b, float* o, void* ws, hipStream_t s) {
    if (g.D != pf::D || g.Hv / g.Hk > 8)
        return hipErrorNotSupported;
    const int SP = static_cast<int>(pf::seg_pitch(T));
    const pf::Ws W = pf::carve(ws, g.B, g.Hk, g.Hv, SP);
    const int G = g.Hv / g.Hk;
    const int units = g.B * g.Hk;
    const int scan_grid = 8 * ((units + 7) / 8) * G * pf::NS;
    const dim3 block(256);
    for (int seg0 = 0; seg0 < T; seg0 += pf::SEG) {
        const int len = std::min(pf::SEG, T - seg0);
        const int nch = (len + pf::CH - 1) / pf::CH;
        const int nblk = nch * (pf::CH / pf::TB);
        const int chunks = g.B * g.Hk * nch;
        const dim3 cgrid(static_cast<unsigned>(8 * ((chunks + 7) / 8) * (pf::CH / pf::TB)));
        const dim3 cblock(static_cast<unsigned>(((2 + G) * pf::D / 2 + kWave - 1) / kWave * kWave));
        if (g.bf16)
            hipLaunchKernelGGL(pf::conv_kernel<uint16_t>, cgrid, cblock, 0, s, static_cast<const uint16_t*>(x),
                               static_cast<const uint16_t*>(tail), static_cast<const uint16_t*>(w), W, T, seg0, SP,
                               nblk, g.B, g.Hk, g.Hv, g.C);
        else
            hipLaunchKernelGGL(pf::conv_kernel<float>, cgrid, cblock, 0, s, static_cast<const float*>(x),
                               static_cast<const float*>(tail), static_cast<const float*>(w), W, T, seg0, SP, nblk,
                               g.B, g.Hk, g.Hv, g.C);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(pf::tri_kernel, dim3(static_cast<unsigned>(g.B * g.Hv * nch)), block, 0, s, a, b, W, T,
                           seg0, SP, nch, g.Hk, g.Hv);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
        hipLaunchKernelGGL(pf::scan_kernel, dim3(static_cast<unsigned>(scan_grid)), dim3(512), 0, s, S, o, W, T,
                           seg0, SP, nch, g.B, g.Hk, g.Hv);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    const int64_t total = static_cast<int64_t>(g.B) * g.C;
    const dim3 tgrid(static_cast<unsigned>((total + 255) / 256));
    if (g.bf16)
        hipLaunchKernelGGL(pf::tail_kernel<uint16_t>, tgrid, block, 0, s, static_cast<const uint16_t*>(x),
                           static_cast<uint16_t*>(tail), T, g.C, total);
    else
        hipLaunchKernelGGL(pf::tail_kernel<float>, tgrid, block, 0, s, static_cast<const float*>(x),
                           static_cast<float*>(tail), T, g.C, total);
    return hipGetLastError();
}

}  // namespace gdn
