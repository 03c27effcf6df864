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
// Work split for MI355X, per segment of at most 4,096 tokens, every chunk
// product on fp16 MFMAs (fp32 accumulation):
//   conv  (parallel over 32-token blocks x q/k heads): conv + SiLU of the
//         q/k head's channels and of its value heads' channels, q/k L2 norm;
//         writes fp16 q^, k^, k^ transposed and v transposed, as fragments.
//   tri   (parallel over value heads x chunks): gates and G, K K^T and K Q^T,
//         A, the blocked inverse T in fp32 (16x16 diagonal blocks by
//         substitution, off-diagonal blocks by fp32 MFMA block products), then
//         U~ = T (beta V) and W~^T = (beta e^G K)^T T^T.  P, U~ and W~ are
//         written straight from registers, with e^G and e^{G_n - G}.
//   scan  (sequential over chunks; one workgroup per (sequence, value head,
//         32-row slice of the state)): Z = W~ S0^T, U = U~ - Z,
//         O = s (e^G (.) Q S0^T + P U), S <- e^{G_n} S + (e^{G_n - G} (.) U)^T K.
//         The state is held transposed in accumulator tiles, so the
//         recurrence passes from one product to the next in registers.
// The workspace holds one segment (about 228 MB at the 27B-class shape),
// whatever the prompt length, small enough to live in the Infinity Cache.
#include <algorithm>
#include <utility>

#include "gdn_core.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace pf {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int D = 128;       // head width handled by the prefill kernels
constexpr int CH = 64;       // chunk length
// Tokens per segment: the workspace of one segment (about 228 MB at the
// 27B-class shape) still fits the 256 MB Infinity Cache between its writes
// (conv, tri) and its reads (tri, scan).  Measured on that layer at T = 32,768:
// 1,226-1,278 us at 4,096 against 1,363 at 2,048, 1,570 at 1,024 and 1,586 at
// 8,192 (whose workspace no longer fits).
constexpr int SEG = 4096;
constexpr int TB = 16;       // tokens per conv sub-block (one k-step of a chunk)
constexpr int DS = 32;       // state rows per scan workgroup
constexpr int NS = D / DS;   // scan workgroups per value head
constexpr int MP = CH + 1;   // fp32 pitch of A (a 64x64 matrix) in LDS
constexpr int TP = CH + 4;   // fp32 pitch of T in LDS: rows 16-byte aligned
constexpr float kScale = Scale<D>::value;

// Workspace of one segment; SP = token pitch (segment length rounded to 64),
// NC = SP / 64 chunks.  Chunk matrices are stored in the order the 32x32x16
// MFMAs read them (frag_base / acc_base below), so that each wave's operand
// load is one contiguous run of 64 lanes x 16 bytes:
//   q, k  fp16 [B][Hk][NC][fragments of 64 tokens x 128 keys]   q^, k^ (zero past the prompt)
//   kt    fp16 [B][Hk][NC][fragments of 128 keys x 64 tokens]   k^ transposed
//   vt    fp16 [B][Hv][NC][fragments of 128 dims x 64 tokens]   v transposed
//   ut    fp16 [B][Hv][NC][accumulators of 64 tokens x 128 dims] U~ = T (beta V)
//   wt    fp16 [B][Hv][NC][fragments of 64 tokens x 128 keys]   W~ = T (beta e^G K)
//   P     fp16 [B][Hv][NC][fragments of 64 x 64 tokens]
//   eg    f32  [B][Hv][SP]                     e^{G_t}
//   ed    f32  [B][Hv][SP]                     e^{G_last - G_t} of the token's chunk
struct Ws {
    _Float16 *q, *k, *kt, *vt, *ut, *wt, *P;
    float *eg, *ed;
};

inline size_t seg_pitch(int T) { return static_cast<size_t>(T >= SEG ? SEG : (T + CH - 1) / CH * CH); }

inline size_t ws_bytes(int B, int Hk, int Hv, size_t SP) {
    const size_t per_tok = 3ull * Hk * D * 2 + 3ull * Hv * D * 2 + Hv * CH * 2ull + 2ull * Hv * 4;
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
    w.ed = take32(ng);
    return w;
}

__device__ __forceinline__ h8 ld8(const _Float16* p) { return *reinterpret_cast<const h8*>(p); }

// 32x32x16 fp16 MFMA.  Lane (hi, c) = (lane / 32, lane % 32).  A fragment: row c,
// eight k values; B fragment: column c, the same eight k; accumulator v of lane
// (hi, c) is row 8 (v / 4) + 4 hi + v % 4, column c.
__device__ __forceinline__ f16v mma32(h8 a, h8 b, f16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 zero4() { return f4{0.0f, 0.0f, 0.0f, 0.0f}; }
__device__ __forceinline__ f16v zero16() {
    f16v z;
#pragma unroll
    for (int v = 0; v < 16; ++v)
        z[v] = 0.0f;
    return z;
}

// Fragment order of a chunk matrix M[row][k].  Tiles of 32 rows x 16 k follow
// one another (nks k-steps per row tile), each 64 lanes x 8 fp16.  Slot e of
// lane half hi holds k = kperm(hi, e) of its k-step rather than 8 hi + e: the
// accumulator values 8 s' .. 8 s' + 7 of a 32 x 32 product are exactly the rows
// 16 s' + kperm(hi, e), so a product's accumulators feed the next product's B
// operand in registers, with the other operand stored in this order.  A
// contraction is indifferent to the order of its k, so the same storage serves
// as A fragment (rows as M) and as B fragment (rows as N).
__host__ __device__ constexpr int kperm(int hi, int e) { return ((e >> 2) << 3) + 4 * hi + (e & 3); }
__device__ __forceinline__ int frag_base(int row, int ks, int nks, int hi) {
    return ((((row >> 5) * nks + ks) * 64) + hi * 32 + (row & 31)) * 8;
}
// Accumulator order of M[row][col] (32 x 32 tiles, nct per row of tiles):
// lane (hi, c) holds the 16 values of its accumulator, fp16, contiguously.
__device__ __forceinline__ int acc_base(int rt, int ct, int nct, int lane) { return ((rt * nct + ct) * 64 + lane) * 16; }
// Fragment `tile` of a fragment-ordered matrix: one contiguous 1 KB run per wave.
__device__ __forceinline__ h8 ldfrag(const _Float16* m, int tile, int lane) { return ld8(m + tile * 512 + lane * 8); }
// The same for a fragment read once (non-temporal: it need not stay cached).
__device__ __forceinline__ h8 ldfrag_once(const _Float16* m, int tile, int lane) {
    return __builtin_nontemporal_load(reinterpret_cast<const h8*>(m + tile * 512 + lane * 8));
}
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

// Two adjacent channels of one token, loaded together.
template <typename Act>
struct Pair;
template <>
struct Pair<uint16_t> {
    using raw = uint32_t;
    __device__ static raw load(const uint16_t* p) { return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p)); }
    __device__ static raw make(uint16_t a, uint16_t b) { return a | (static_cast<uint32_t>(b) << 16); }
    __device__ static float lo(raw v) { return __uint_as_float(v << 16); }
    __device__ static float hi(raw v) { return __uint_as_float(v & 0xFFFF0000u); }
};
template <>
struct Pair<float> {
    using raw = float2;
    __device__ static raw load(const float* p) {
        typedef float f2 __attribute__((ext_vector_type(2)));
        const f2 v = __builtin_nontemporal_load(reinterpret_cast<const f2*>(p));
        return make_float2(v.x, v.y);
    }
    __device__ static raw make(float a, float b) { return make_float2(a, b); }
    __device__ static float lo(raw v) { return v.x; }
    __device__ static float hi(raw v) { return v.y; }
};

constexpr int SUB = 1;   // 16-token sub-blocks per conv workgroup

// One workgroup per (sequence, q/k head, SUB x 16 tokens), one thread per pair
// of adjacent channels of the head's group (q, k and its value heads).  Every
// window load of the workgroup is issued before the first is used.  With one
// sub-block per workgroup there are more workgroups than fit on the CUs at
// once, so later ones load while earlier ones compute and write (a segment's
// conv 26.4 -> 24.1 us against two sub-blocks, whose grid was resident at
// once and moved through load, compute and write in step).
template <typename Act>
__global__ __launch_bounds__(640) void conv_kernel(const Act* __restrict__ x, const Act* __restrict__ tail,
                                                   const Act* __restrict__ w, Ws ws, int T, int seg0, int SP,
                                                   int nch, int B, int Hk, int Hv, int C) {
    __shared__ __align__(16) float ys[TB][2 * D];    // q~ | k~ of a sub-block, fp32
    __shared__ __align__(16) _Float16 qkh[2][TB][D]; // q^, k^ of a sub-block, fp16
    // The workgroups of one chunk write the two halves of the same q^ / k^
    // fragments; they share an XCD (blockIdx % 8 picks it).  The q/k head
    // varies fastest, so the workgroups resident together read whole token
    // rows of x rather than one head's pieces of many rows (a segment's conv
    // 40.3 -> 38.0 us against chunk-fastest order).
    constexpr int BPC = CH / (SUB * TB);             // workgroups per chunk
    const int xcd = blockIdx.x % 8, r8 = blockIdx.x / 8;
    const int chunk_id = (r8 / BPC) * 8 + xcd;       // (sequence, chunk of the segment, q/k head)
    if (chunk_id >= B * Hk * nch)
        return;
    const int g = chunk_id % Hk;
    const int cl = (chunk_id / Hk) % nch;
    const int bq = chunk_id / (nch * Hk);
    const int cb = (r8 % BPC) * SUB * TB;            // chunk offset of the workgroup's first token
    const int t0 = seg0 + cl * CH + cb;              // its prompt index
    const int G = Hv / Hk;
    const int NC = SP / CH;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const Act* xb = x + static_cast<size_t>(bq) * T * C;
    const Act* tbq = tail + static_cast<size_t>(bq) * C * 4;
    const int npair = (2 + G) * D / 2;
    const bool active = static_cast<int>(threadIdx.x) < npair;
    const int ch = 2 * (active ? static_cast<int>(threadIdx.x) : npair - 1);   // first channel in the group
    const int cg = ch < D ? g * D + ch : ch < 2 * D ? Hk * D + g * D + (ch - D) : 2 * Hk * D + G * g * D + (ch - 2 * D);
    using P = Pair<Act>;
    float wf0[4], wf1[4];
    Quad<Act>::to_float(Quad<Act>::load(w + static_cast<size_t>(cg) * 4), wf0);
    Quad<Act>::to_float(Quad<Act>::load(w + static_cast<size_t>(cg + 1) * 4), wf1);
    typename P::raw hist[SUB * TB + 3];
    if (t0 >= 3) {
#pragma unroll
        for (int m = 0; m < SUB * TB + 3; ++m) {
            const int t = t0 + m - 3;
            hist[m] = P::load(xb + static_cast<size_t>(t < T ? t : T - 1) * C + cg);
        }
    } else {   // the prompt's first tokens: the window reaches into the tail
#pragma unroll
        for (int m = 0; m < SUB * TB + 3; ++m) {
            const int t = t0 + m - 3;
            hist[m] = t < 0 ? P::make(tbq[static_cast<size_t>(cg) * 4 + 4 + t], tbq[static_cast<size_t>(cg + 1) * 4 + 4 + t])
                            : P::load(xb + static_cast<size_t>(t < T ? t : T - 1) * C + cg);
        }
    }
    const size_t qkc = ((static_cast<size_t>(bq) * Hk + g) * NC + cl) * kChunkQK;
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb) {
        const int co = cb + sb * TB;                 // chunk offset of the sub-block's first token
        const int ks = co / TB;                      // the sub-block's tokens are k-step ks of the chunk
        float y0[TB], y1[TB];
#pragma unroll
        for (int j = 0; j < TB; ++j) {
            float w0[4], w1[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                w0[m] = P::lo(hist[sb * TB + j + m]);
                w1[m] = P::hi(hist[sb * TB + j + m]);
            }
            const bool valid = t0 + sb * TB + j < T;
            y0[j] = valid ? conv_silu_fast(wf0, w0) : 0.0f;
            y1[j] = valid ? conv_silu_fast(wf1, w1) : 0.0f;
        }
        if (active) {
            if (ch < 2 * D) {
#pragma unroll
                for (int j = 0; j < TB; ++j)
                    *reinterpret_cast<float2*>(&ys[j][ch]) = make_float2(y0[j], y1[j]);
            } else {
                // v^T: rows d and d + 1, k = token; this thread owns both lane halves of each row
                const int h = G * g + (ch - 2 * D) / D;
                const int d = (ch - 2 * D) % D;
                _Float16* vc = ws.vt + ((static_cast<size_t>(bq) * Hv + h) * NC + cl) * kChunkQK;
#pragma unroll
                for (int hi = 0; hi < 2; ++hi) {
                    h8 v0, v1;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        v0[e] = static_cast<_Float16>(y0[kperm(hi, e)]);
                        v1[e] = static_cast<_Float16>(y1[kperm(hi, e)]);
                    }
                    *reinterpret_cast<h8*>(vc + frag_base(d, ks, CH / 16, hi)) = v0;
                    *reinterpret_cast<h8*>(vc + frag_base(d + 1, ks, CH / 16, hi)) = v1;
                }
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
        // q^, k^: row = token co + tl, k = key; slot group (hi) of key step s holds
        // keys 16 s + 4 hi .. + 3 and 16 s + 8 + 4 hi .. + 3.
        for (int idx = threadIdx.x; idx < 2 * (D / 16) * 2 * TB; idx += blockDim.x) {
            const int tl = idx % TB, hi = (idx / TB) & 1, s = (idx / (2 * TB)) % (D / 16), which = idx / (D / 16 * 2 * TB);
            const h4 lo = *reinterpret_cast<const h4*>(&qkh[which][tl][16 * s + 4 * hi]);
            const h4 up = *reinterpret_cast<const h4*>(&qkh[which][tl][16 * s + 8 + 4 * hi]);
            const h8 v = {lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
            *reinterpret_cast<h8*>((which ? ws.k : ws.q) + qkc + frag_base(co + tl, s, D / 16, hi)) = v;
        }
        // k^T: row = key, k = token
        for (int idx = threadIdx.x; idx < 2 * D; idx += blockDim.x) {
            const int key = idx % D, hi = idx / D;
            h8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = qkh[1][kperm(hi, e)][key];
            *reinterpret_cast<h8*>(ws.kt + qkc + frag_base(key, ks, CH / 16, hi)) = v;
        }
        if (sb + 1 < SUB)
            __syncthreads();   // ys and qkh are reused by the next sub-block
    }
}

// ------------------------------------------------------------ tri

struct alignas(16) TriSmem {
    float T[CH][TP];              // (I + A)^-1; rows 16-byte aligned for the fragment reads
    float A[CH][MP];
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
    const int hi = lane >> 5, c32 = lane & 31;
    const size_t hs = (static_cast<size_t>(bq) * Hv + h) * SP + s0;   // this head's token row base

    // Gate inputs first, then every operand fragment this wave needs, so that
    // waiting for the gates does not wait for the fragments.
    float av = 0.0f, bv = 0.0f;
    if (wave == 0 && lane < n) {
        const size_t idx = (static_cast<size_t>(bq) * T + t_base + lane) * Hv + h;
        av = a[idx];
        bv = bg[idx];
    }
    // 32 x 32 token tiles (m, n) of K K^T and K Q^T (m: tile of k as rows, n:
    // tile of k or q as columns; only m <= n is needed):
    //   wave 0: KK(0,0), KQ(0,0);  wave 1: KK(0,1);  wave 2: KQ(0,1);  wave 3: KK(1,1), KQ(1,1).
    // Then U~ and W~: wave w owns value column tile w and key tile w.
    const int mt = wave == 3 ? 1 : 0;
    const int nt = wave == 0 ? 0 : 1;
    const size_t qkc = ((static_cast<size_t>(bq) * Hk + g) * NC + cl) * kChunkQK;
    const size_t hc = ((static_cast<size_t>(bq) * Hv + h) * NC + cl) * kChunkQK;
    const _Float16* kA = ws.k + qkc;
    const _Float16* kB = (wave == 1 ? ws.k : ws.q) + qkc;
    h8 fa[8], fb[8], vf[4], kf[4];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        fa[s] = ldfrag(kA, mt * 8 + s, lane);
        fb[s] = ldfrag(kB, nt * 8 + s, lane);
    }
    // upper blocks of T are zero (the diagonal blocks are written whole below)
    for (int e = threadIdx.x; e < 6 * 256; e += blockDim.x) {
        const int blk = e / 256, r = (e / 16) % 16, c = e % 16;
        const int I = blk < 3 ? 0 : blk < 5 ? 1 : 2;
        const int J = blk < 3 ? blk + 1 : blk < 5 ? blk - 1 : 3;
        sm.T[16 * I + r][16 * J + c] = 0.0f;
    }

    // gates first in program order: their inputs were requested first
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
        const float eg = __builtin_amdgcn_exp2f(l2);
        const float ed = __builtin_amdgcn_exp2f(__shfl(l2, kWave - 1, kWave) - l2);
        sm.G[lane] = l2;
        sm.beta[lane] = be;
        sm.bv[lane] = be;
        sm.bk[lane] = be * eg;
        ws.eg[hs + lane] = eg;
        ws.ed[hs + lane] = ed;
    }
    f16v kk = zero16(), kq = zero16();
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        if (wave == 1) {
            kk = mma32(fa[s], fb[s], kk);
        } else {
            if (wave != 2)
                kk = mma32(fa[s], fa[s], kk);
            kq = mma32(fa[s], fb[s], kq);
        }
    }

    // v and k^T fragments are needed only after the inverse: requested once
    // the products have freed fa / fb, which keeps the workgroup at 4 per CU
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        vf[s] = ldfrag_once(ws.vt + hc, wave * 4 + s, lane);   // v^T of this value head: read once
        kf[s] = ldfrag(ws.kt + qkc, wave * 4 + s, lane);
    }
    __syncthreads();

    // Accumulator v of tile (mt, nt) is row t' = 32 mt + 8 (v / 4) + 4 hi + v % 4
    // (k side), column t = 32 nt + c32 (k or q side).
    {
        const int t = 32 * nt + c32;
        const float gt = sm.G[t], bt = sm.beta[t];
        if (wave != 2) {
            // A[t][t'] = beta_t e^{G_t - G_t'} k_t . k_t' for t > t'
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int tp = 32 * mt + 8 * (v >> 2) + 4 * hi + (v & 3);
                if (t > tp)
                    sm.A[t][tp] = bt * __builtin_amdgcn_exp2f(gt - sm.G[tp]) * kk[v];
            }
        }
        _Float16* Pc = ws.P + ((static_cast<size_t>(bq) * Hv + h) * NC + cl) * kChunkP;
        if (wave != 1) {
            // P[t][t'] = e^{G_t - G_t'} q_t . k_t' for t >= t': the accumulators
            // 8 j .. 8 j + 7 are P's fragment (row tile nt, k-step 2 mt + j)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                h8 p;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int v = 8 * j + e;
                    const int tp = 32 * mt + 8 * (v >> 2) + 4 * hi + (v & 3);
                    p[e] = static_cast<_Float16>(t >= tp ? __builtin_amdgcn_exp2f(gt - sm.G[tp]) * kq[v] : 0.0f);
                }
                *reinterpret_cast<h8*>(Pc + ((nt * 4 + 2 * mt + j) * 64 + lane) * 8) = p;
            }
        } else {
            // P's fragments (row tile 0, k-steps 2, 3) lie above the diagonal
            const h8 zero = {};
#pragma unroll
            for (int j = 0; j < 2; ++j)
                *reinterpret_cast<h8*>(Pc + ((2 + j) * 64 + lane) * 8) = zero;
        }
    }
    __syncthreads();

    // diagonal 16x16 blocks of (I + A)^-1: wave 0, lane = (block, column)
    if (wave == 0) {
        const int o = 16 * (lane >> 4), j = lane & 15;
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
    // off-diagonal blocks, one block diagonal at a time: T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ.
    // Wave I computes block (I, I - lvl) on fp32 16x16x4 MFMAs, lane (q, c) =
    // (lane / 16, lane % 16).  Step s of a product takes k = 4 q + s, so the
    // accumulators of Z = sum A_IK T_KJ (lane (q, c): rows 4 q .. 4 q + 3, column
    // c) are directly the B operand of -T_II Z.  One barrier per level.
    {
        const int q = lane >> 4, c = lane & 15;
        for (int lvl = 1; lvl < 4; ++lvl) {
            if (wave >= lvl) {
                const int I = wave, J = wave - lvl;
                f4 z = zero4();
                for (int K = J; K < I; ++K)
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        z = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.A[16 * I + c][16 * K + 4 * q + s],
                                                                 sm.T[16 * K + 4 * q + s][16 * J + c], z, 0, 0, 0);
                f4 t = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    t = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.T[16 * I + c][16 * I + 4 * q + s], z[s], t, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sm.T[16 * I + 4 * q + r][16 * J + c] = -t[r];
            }
            __syncthreads();
        }
    }

    // T as fragments (row tile tt, k-step s over t'); the same registers are
    // T's A fragment for U~ and T^T's B fragment for W~^T.
    h8 tf[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const f4 lo = *reinterpret_cast<const f4*>(&sm.T[32 * tt + c32][16 * s + 4 * hi]);
            const f4 up = *reinterpret_cast<const f4*>(&sm.T[32 * tt + c32][16 * s + 8 + 4 * hi]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                tf[tt][s][e] = static_cast<_Float16>(lo[e]);
                tf[tt][s][4 + e] = static_cast<_Float16>(up[e]);
            }
        }
    // beta V (column tile w) and beta e^G K (key tile w) with the token as k
    h8 vs[4], ks[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int tp = 16 * s + kperm(hi, e);
            vs[s][e] = static_cast<_Float16>(static_cast<float>(vf[s][e]) * sm.bv[tp]);
            ks[s][e] = static_cast<_Float16>(static_cast<float>(kf[s][e]) * sm.bk[tp]);
        }
    }
    _Float16* uto = ws.ut + hc;
    _Float16* wto = ws.wt + hc;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        f16v u = zero16(), wv = zero16();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u = mma32(tf[tt][s], vs[s], u);    // U~[t][d]:  rows t (tile tt), columns d (tile w)
            wv = mma32(ks[s], tf[tt][s], wv);  // W~^T[key][t]: rows key (tile w), columns t (tile tt)
        }
        // U~ in accumulator order
        h8 u0, u1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            u0[e] = static_cast<_Float16>(u[e]);
            u1[e] = static_cast<_Float16>(u[8 + e]);
        }
        _Float16* up = uto + acc_base(tt, wave, D / 32, lane);
        *reinterpret_cast<h8*>(up) = u0;
        *reinterpret_cast<h8*>(up + 8) = u1;
        // W~^T's accumulators 8 j .. 8 j + 7 are W~'s fragment (row tile tt, key step 2 w + j)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            h8 f;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                f[e] = static_cast<_Float16>(wv[8 * j + e]);
            *reinterpret_cast<h8*>(wto + ((tt * (D / 16) + 2 * wave + j) * 64 + lane) * 8) = f;
        }
    }
}

// ------------------------------------------------------------ scan

// One workgroup per (sequence, value head, 32-row slice of the state), six
// waves with one barrier per chunk:
//   state  (waves 0, 1: rows 16 w .. 16 w + 15 of the slice) hold S^T of their
//          rows (keys x rows) in eight 16 x 16 accumulator tiles across chunks
//          and run the recurrence on 16x16x32 fp16 MFMAs:
//            Z = W~ S0^T - U~        (the accumulators start at -U~: Z = -U)
//            S^T <- e^{G_n} S^T + K^T (e^{G_n - G} (.) U)
//          The fp16 copies of S^T's accumulators are directly the B fragments
//          of Z, and Z's accumulators, negated and scaled per token, directly
//          the B fragments of the update: no LDS round trip and no barrier
//          inside the recurrence.  Each wave hands S0^T and U of its rows to
//          the output waves through LDS (two buffers).
//   output (waves 2, 3: token tile 32 (w - 2)) compute Y = Q S0^T and P U one
//          chunk behind on 32x32x16 MFMAs and store o = s (e^G Y + P U); Q and
//          P stream through a register ring.
//   copies (waves 4, 5) copy the q/k head's k^T, this slice's U~, e^G and
//          e^{G_n - G} of chunk k + 2 and W~ of chunk k + 3 into a three-stage
//          LDS ring by direct global-to-LDS loads, and wait for the previous
//          group before the barrier that ends step k.  Two waves share the
//          copies so that two groups' worth stays within each wave's
//          outstanding vector loads.
// Splitting the rows over two waves halves the matrix and vector work on the
// recurrence's dependent chain; each state wave still reads the whole chunk's
// W~ and k^T (32 KB) from LDS, k^T one read behind each product of Z and the
// next chunk's W~ one read behind each product of the update (hence W~ one
// chunk ahead in the ring).
// Workgroups of one (sequence, q/k head) share an XCD and its L2.
constexpr int kStages = 3;
constexpr int kOutRing = 2;
constexpr int kScanThreads = 6 * kWave;

struct alignas(16) ScanSmem {
    h8 wt[kStages][16][64];     // W~ fragments (token tile, key step)
    h8 kt[kStages][16][64];     // k^T fragments of the q/k head (key tile, token step)
    h8 ut[kStages][2][64][2];   // U~ of the slice: token tile, lane, 32 bytes
    float eg[kStages][CH];
    float ed[kStages][CH];
    h8 xs[2][8][64];            // S0^T as 32x32x16 B fragments (key step)
    h8 xu[2][4][64];            // U as 32x32x16 B fragments (token step)
};

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 16x16x32 fp16 MFMA.  Lane (q, r) = (lane / 16, lane % 16).  A fragment: row r,
// eight k values; B fragment: column r, the same eight k; accumulator i of lane
// (q, c) is row 4 q + i, column c.
__device__ __forceinline__ f4 mma16(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

// Row m of the recurrence's 16-row tile t (keys: t = 0..7; tokens: t = 0..3)
// is index rho(t, m) of the chunk.  The eight indices that a lane of quarter q
// contributes to k-step s (rows 4 q .. 4 q + 3 of tiles 2 s and 2 s + 1) are
// then 16 (2 s + q / 2) + kperm(q % 2, e), e = 0..7: exactly the 16-byte unit
// (k-step 2 s + q / 2, lane half q % 2) of the 32x32x16 fragment storage.  So
// every operand of the recurrence is one 16-byte LDS read per lane from the
// storage the other kernels write, accumulators pass from one product to the
// next in registers, and S0^T and U reach the output waves unit for unit in
// their 32x32x16 B layout.
__host__ __device__ constexpr int rho(int t, int m) {
    return 32 * (t >> 1) + 16 * (m >> 3) + 8 * (t & 1) + 4 * ((m >> 2) & 1) + (m & 3);
}
constexpr bool rho_is_a_permutation() {
    bool seen[D] = {};
    for (int t = 0; t < D / 16; ++t)
        for (int m = 0; m < 16; ++m) {
            const int r = rho(t, m);
            if (r < 0 || r >= D || seen[r])
                return false;
            seen[r] = true;
        }
    for (int s = 0; s < D / 32; ++s)
        for (int q = 0; q < 4; ++q)
            for (int e = 0; e < 8; ++e)
                if (rho(2 * s + (e >> 2), 4 * q + (e & 3)) != 16 * (2 * s + (q >> 1)) + kperm(q & 1, e))
                    return false;
    return true;
}
static_assert(rho_is_a_permutation(), "the recurrence's row order must tile the chunk's 32x32x16 fragment units");

struct OutOps {
    h8 qf[8], pf[4];
    f4 eg[4];
};

__global__ __launch_bounds__(kScanThreads) void scan_kernel(float* __restrict__ S, float* __restrict__ o, Ws ws,
                                                            int T, int seg0, int SP, int nch, int B, int Hk, int Hv) {
    __shared__ ScanSmem sm;
    const int G = Hv / Hk;
    // workgroups of one (sequence, q/k head) share an XCD: blockIdx % 8 picks the XCD
    const int xcd = blockIdx.x % 8, r8 = blockIdx.x / 8;
    const int gu = (r8 / (G * NS)) * 8 + xcd;
    if (gu >= B * Hk)
        return;
    const int rem = r8 % (G * NS);
    const int bq = gu / Hk, g = gu % Hk, h = G * g + rem / NS, slc = rem % NS, row0 = slc * DS;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int hi = lane >> 5, c32 = lane & 31;
    const int NC = SP / CH;
    const size_t hbase = (static_cast<size_t>(bq) * Hv + h) * SP;   // token rows of value head h
    const size_t vbase = (static_cast<size_t>(bq) * Hv + h) * NC;   // chunks of value head h
    const size_t kbase = (static_cast<size_t>(bq) * Hk + g) * NC;   // chunks of q/k head g
    const int len = min(SEG, T - seg0);

    if (wave >= 4) {
        // ---- copies, in groups: group j (j = -1 .. nch - 1) is W~ of chunk j + 1
        // with e^G and e^{G_n - G} of chunk j (wave 4) and k^T and U~ of chunk j
        // (wave 5), in ring slot (j + 3) % 3.  The state waves read group j's
        // k^T during step j's Z and its W~ during step j's update, so W~ runs one
        // chunk ahead of the rest.  Each wave's copies of two groups fit its 63
        // outstanding vector loads.
        auto count = [&](int j) {   // copies this wave issues for group j
            return wave == 4 ? (j + 1 < nch ? 16 : 0) + (j >= 0 ? 2 : 0) : (j >= 0 ? 20 : 0);
        };
        auto issue = [&](int j) {
            const int st = (j + kStages) % kStages;
            if (wave == 4) {
                if (j + 1 < nch) {
                    const char* wsrc = reinterpret_cast<const char*>(ws.wt + (vbase + j + 1) * kChunkQK) + lane * 16;
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        __builtin_amdgcn_global_load_lds(wsrc + i * 1024, &sm.wt[st][i][0], 16, 0, 0);
                }
                if (j >= 0) {
                    __builtin_amdgcn_global_load_lds(ws.eg + hbase + j * CH + lane, &sm.eg[st][0], 4, 0, 0);
                    __builtin_amdgcn_global_load_lds(ws.ed + hbase + j * CH + lane, &sm.ed[st][0], 4, 0, 0);
                }
            } else if (j >= 0) {
                const char* ksrc = reinterpret_cast<const char*>(ws.kt + (kbase + j) * kChunkQK) + lane * 16;
                const char* usrc = reinterpret_cast<const char*>(ws.ut + (vbase + j) * kChunkQK) + lane * 16;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    __builtin_amdgcn_global_load_lds(ksrc + i * 1024, &sm.kt[st][i][0], 16, 0, 0);
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)   // accumulator tile (tt, slc) of U~: 2 KB
                        __builtin_amdgcn_global_load_lds(usrc + (tt * (D / 32) + slc) * 2048 + h2 * 1024,
                                                         &sm.ut[st][tt][0][0] + h2 * 64, 16, 0, 0);
            }
        };
        // wait until at most n of this wave's copies are in flight
        auto wait_pending = [&](int n) {
            switch (n) {
            case 2: wait_vmem<2>(); break;
            case 18: wait_vmem<18>(); break;
            case 20: wait_vmem<20>(); break;
            default: wait_vmem<0>(); break;
            }
        };
        issue(-1);
        issue(0);
        if (nch > 1)
            issue(1);
        wait_pending(nch > 1 ? count(1) : 0);
        __builtin_amdgcn_s_barrier();
        for (int k = 0; k < nch; ++k) {
            if (k + 2 < nch)
                issue(k + 2);
            wait_pending(k + 2 < nch ? count(k + 2) : 0);
            __builtin_amdgcn_s_barrier();
        }
        __builtin_amdgcn_s_barrier();
    } else if (wave < 2) {
        // ---- state: rows row0 + 16 wave + c
        const int q = lane >> 4, c = lane & 15, qs = q >> 1;
        float* Sh = S + ((static_cast<size_t>(bq) * Hv + h) * D + row0 + 16 * wave + c) * D;
        f4 st[8];   // st[t][i]: key rho(t, 4 q + i)
#pragma unroll
        for (int t = 0; t < 8; ++t)
            st[t] = *reinterpret_cast<const f4*>(Sh + rho(t, 4 * q));
        // LDS lane positions: an A fragment row rho(t, c) sits at lane (q % 2) * 32
        // + rho(t, c) % 32 of its 1 KB run (which depends on t only through t % 2);
        // this wave's B units for the output waves at (q % 2) * 32 + 16 wave + c.
        const int la0 = (q & 1) * 32 + (rho(0, c) & 31), la1 = (q & 1) * 32 + (rho(1, c) & 31);
        const int xl = (q & 1) * 32 + 16 * wave + c;
        h8 wf[4][4];   // W~ of the current chunk: token tile T, key step s
        auto read_wt = [&](int slot) {
#pragma unroll
            for (int T4 = 0; T4 < 4; ++T4)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    wf[T4][s] = sm.wt[slot][(T4 >> 1) * 8 + 2 * s + qs][(T4 & 1) ? la1 : la0];
        };
        __syncthreads();
        read_wt(kStages - 1);   // W~ of chunk 0 (copy group -1)
        for (int k = 0; k < nch; ++k) {
            const int stg = k % kStages, par = k & 1;
            // token rho(T, 4 q + i) of U~'s accumulator tile T / 2 is value 8 (q / 2) + 4 (T % 2) + i of lane xl
            const h8 u0 = sm.ut[stg][0][xl][qs], u1 = sm.ut[stg][1][xl][qs];
            const float eglast = sm.eg[stg][CH - 1];
            f4 edv[2][2];  // e^{G_n - G} of the tokens of update step s2, slots 4 j .. 4 j + 3
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    edv[s2][j] = *reinterpret_cast<const f4*>(&sm.ed[stg][16 * (2 * s2 + qs) + 8 * j + 4 * (q & 1)]);
            __builtin_amdgcn_sched_barrier(0);
            h8 bs[4];
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    bs[s][e] = static_cast<_Float16>(st[2 * s + (e >> 2)][e & 3]);
            f4 z[4];
#pragma unroll
            for (int T4 = 0; T4 < 4; ++T4)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    z[T4][i] = -static_cast<float>((T4 >> 1 ? u1 : u0)[4 * (T4 & 1) + i]);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int T4 = 0; T4 < 4; ++T4)
                    z[T4] = mma16(wf[T4][s], bs[s], z[T4]);
            // k^T is read while Z is in the matrix pipe
            h8 kf[8][2];   // key tile t, token step s2
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    kf[t][s2] = sm.kt[stg][(t >> 1) * 4 + 2 * s2 + qs][(t & 1) ? la1 : la0];
#pragma unroll
            for (int t = 0; t < 8; ++t)
                st[t] *= eglast;
            // S0^T for the output waves, off the recurrence's path
#pragma unroll
            for (int s = 0; s < 4; ++s)
                sm.xs[par][2 * s + qs][xl] = bs[s];
            // each k^T read issues behind one of Z's products
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            // U = -Z; token step s2 of U is tiles 2 s2 and 2 s2 + 1
            h8 bu[2], bd[2];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float u = -z[2 * s2 + (e >> 2)][e & 3];
                    bu[s2][e] = static_cast<_Float16>(u);
                    bd[s2][e] = static_cast<_Float16>(u * edv[s2][e >> 2][e & 3]);
                }
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    st[t] = mma16(kf[t][s2], bd[s2], st[t]);
            // the next chunk's W~ (copy group k) is read while the update is in the
            // matrix pipe, one read behind each product (after the last chunk the
            // slot holds no W~ and the values read go unused)
            read_wt(stg);
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                sm.xu[par][2 * s2 + qs][xl] = bu[s2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            }
            __syncthreads();
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 8; ++t)
            *reinterpret_cast<f4*>(Sh + rho(t, 4 * q)) = st[t];
    } else {
        // ---- output, token tile tt
        const int tt = wave - 2;
        const uint32_t ostride = static_cast<uint32_t>(Hv) * D;   // a chunk's o (64 rows) spans < 4 G floats
        float* obase = o + ((static_cast<size_t>(bq) * T + seg0) * Hv + h) * D + row0;
        auto load = [&](OutOps& op, int cl) {
            const _Float16* qc = ws.q + (kbase + cl) * kChunkQK;
            const _Float16* pc = ws.P + (vbase + cl) * kChunkP;
#pragma unroll
            for (int s = 0; s < 8; ++s)
                op.qf[s] = ldfrag(qc, tt * 8 + s, lane);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                op.pf[s] = ldfrag(pc, tt * 4 + s, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                op.eg[j] = *reinterpret_cast<const f4*>(ws.eg + hbase + cl * CH + 32 * tt + 8 * j + 4 * hi);
        };
        OutOps ring[kOutRing];
#pragma unroll
        for (int p = 0; p < kOutRing; ++p)
            load(ring[p], min(p, nch - 1));
        __syncthreads();
        __syncthreads();
        auto step = [&](auto pc, int cl) {
            constexpr int P = decltype(pc)::value;
            const OutOps& op = ring[P];
            const int par = cl & 1;
            h8 xs[8], xu[4];
#pragma unroll
            for (int s = 0; s < 8; ++s)
                xs[s] = sm.xs[par][s][lane];
#pragma unroll
            for (int s = 0; s < 4; ++s)
                xu[s] = sm.xu[par][s][lane];
            f16v y = zero16(), pu = zero16();
#pragma unroll
            for (int s = 0; s < 8; ++s)
                y = mma32(op.qf[s], xs[s], y);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                pu = mma32(op.pf[s], xu[s], pu);
            const int n = min(CH, len - cl * CH);
            // the chunk's first row (uniform) and a 32-bit offset per lane and value
            float* orow = obase + static_cast<size_t>(cl) * CH * ostride;
            const uint32_t lrow = static_cast<uint32_t>(32 * tt + 4 * hi) * ostride + c32;
            if (n == CH) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        __builtin_nontemporal_store(kScale * __builtin_fmaf(op.eg[j][r], y[4 * j + r], pu[4 * j + r]),
                                                    orow + (lrow + static_cast<uint32_t>(8 * j + r) * ostride));
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = 32 * tt + 8 * j + 4 * hi + r;
                        if (t < n)
                            __builtin_nontemporal_store(kScale * __builtin_fmaf(op.eg[j][r], y[4 * j + r], pu[4 * j + r]),
                                                        orow + (lrow + static_cast<uint32_t>(8 * j + r) * ostride));
                    }
            }
            load(ring[P], min(cl + kOutRing, nch - 1));
            __syncthreads();
        };
        static_assert(kOutRing == 2, "the ring is walked in pairs");
        int cl0 = 0;
        for (; cl0 + kOutRing <= nch; cl0 += kOutRing) {
            step(std::integral_constant<int, 0>{}, cl0);
            step(std::integral_constant<int, 1>{}, cl0 + 1);
        }
        if (cl0 < nch)
            step(std::integral_constant<int, 0>{}, cl0);
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
        const int chunks = g.B * g.Hk * nch;
        const dim3 cgrid(static_cast<unsigned>(8 * ((chunks + 7) / 8) * (pf::CH / (pf::SUB * pf::TB))));
        const dim3 cblock(static_cast<unsigned>(((2 + G) * pf::D / 2 + kWave - 1) / kWave * kWave));
        if (g.bf16)
            hipLaunchKernelGGL(pf::conv_kernel<uint16_t>, cgrid, cblock, 0, s, static_cast<const uint16_t*>(x),
                               static_cast<const uint16_t*>(tail), static_cast<const uint16_t*>(w), W, T, seg0, SP,
                               nch, g.B, g.Hk, g.Hv, g.C);
        else
            hipLaunchKernelGGL(pf::conv_kernel<float>, cgrid, cblock, 0, s, static_cast<const float*>(x),
                               static_cast<const float*>(tail), static_cast<const float*>(w), W, T, seg0, SP, nch,
                               g.B, g.Hk, g.Hv, g.C);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(pf::tri_kernel, dim3(static_cast<unsigned>(g.B * g.Hv * nch)), block, 0, s, a, b, W, T,
                           seg0, SP, nch, g.Hk, g.Hv);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
        hipLaunchKernelGGL(pf::scan_kernel, dim3(static_cast<unsigned>(scan_grid)), dim3(pf::kScanThreads), 0, s, S,
                           o, W, T, seg0, SP, nch, g.B, g.Hk, g.Hv);
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
