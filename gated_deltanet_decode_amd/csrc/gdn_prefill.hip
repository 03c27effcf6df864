// gdn_prefill.hip -- chunked prefill of a prompt (repository "Architecture"
// page: the prompt is prefilled before the decode loop; CPU page, exactness
// section: the chunked form and the token-by-token form are the same algebra
// and differ only in rounding).
//
// Per value head and chunk of n <= 64 tokens starting from state S0, with
// G_t the inclusive cumulative log-decay inside the chunk (G_t = sum log
// alpha), the recurrence folds into (derivation: the chunk-form test)
//   A    = strict-lower( beta_i e^{G_i - G_j} k_i.k_j ),   T = (I + A)^-1
//   U    = T (beta (.) (V - e^G (.) K S0^T))
//   O    = s ( e^G (.) Q S0^T + P U ),   P = lower-incl( e^{G_i - G_j} q_i.k_j )
//   S_n  = e^{G_n} S0 + U^T (e^{G_n - G} (.) K)
// Only differences G_i - G_j with i >= j are exponentiated.
//
// Work split for MI355X:
//   prep (fully parallel, one workgroup per (sequence, q/k head, chunk)):
//     conv + SiLU of the head's q, k and its G value heads' channels, q/k L2
//     norm, gates and G; K K^T and Q K^T on MFMA (fp16 in, fp32 out), then per
//     value head A, the blocked inverse T in fp32 and P; operands are written
//     as fp16 to a workspace that holds one segment of the prompt.
//   scan (sequential over chunks, one workgroup per (sequence, value head,
//     16-row slice of the state)): the state-dependent products only, all on
//     MFMA 16x16x32 fp16 with fp32 accumulation; the state slice stays in
//     registers in fp32 across chunks.  Workgroups of one q/k group sit on one
//     XCD so they share its L2 for the group's q/k operands.
// Segments of 2,048 tokens bound the workspace (a few tens of MB, independent
// of the prompt length) and keep it small enough for the Infinity Cache.
#include <algorithm>

#include "gdn_core.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace pf {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;       // head width handled by the prefill kernels
constexpr int CH = 64;       // chunk length
constexpr int SEG = 2048;    // tokens per segment
constexpr int DS = 16;       // state rows per scan workgroup
constexpr int NS = D / DS;   // scan workgroups per value head
constexpr int QKP = D + 8;   // fp16 pitch of a q^/k^ row in LDS
constexpr int MP = CH + 1;   // fp32 pitch of a 64x64 matrix row in LDS
constexpr int MAXG = 8;      // value heads per q/k head handled by one prep workgroup
constexpr float kScale = Scale<D>::value;

// Workspace of one segment; SP = token pitch (segment length rounded to 64).
//   q, k  fp16 [B][Hk][SP][D]      normalised q^, k^ (zero past the prompt)
//   kt    fp16 [B][Hk][SP/64][D][64]  k^ transposed per chunk
//   v     fp16 [B][Hv][SP][D]
//   G     f32  [B][Hv][SP]          inclusive cumulative log-decay within the chunk
//   beta  f32  [B][Hv][SP]
//   T, P  fp16 [B][Hv][SP/64][64][64]
struct Ws {
    _Float16 *q, *k, *kt, *v;
    float *G, *beta;
    _Float16 *T, *P;
};

inline size_t seg_pitch(int T) { return static_cast<size_t>(T >= SEG ? SEG : (T + CH - 1) / CH * CH); }

inline size_t ws_bytes(int B, int Hk, int Hv, size_t SP) {
    const size_t per_tok = 3ull * Hk * D * 2 + static_cast<size_t>(Hv) * D * 2 + Hv * 8ull + Hv * 2ull * CH * 2;
    return static_cast<size_t>(B) * SP * per_tok + 256 * 8;
}

inline Ws carve(void* base, int B, int Hk, int Hv, size_t SP) {
    auto align = [](uintptr_t p) { return (p + 255) & ~static_cast<uintptr_t>(255); };
    uintptr_t p = align(reinterpret_cast<uintptr_t>(base));
    Ws w;
    const size_t nqk = static_cast<size_t>(B) * Hk * SP * D, nv = static_cast<size_t>(B) * Hv * SP * D;
    const size_t ng = static_cast<size_t>(B) * Hv * SP, nm = static_cast<size_t>(B) * Hv * SP * CH;
    w.q = reinterpret_cast<_Float16*>(p); p = align(p + nqk * 2);
    w.k = reinterpret_cast<_Float16*>(p); p = align(p + nqk * 2);
    w.kt = reinterpret_cast<_Float16*>(p); p = align(p + nqk * 2);
    w.v = reinterpret_cast<_Float16*>(p); p = align(p + nv * 2);
    w.G = reinterpret_cast<float*>(p); p = align(p + ng * 4);
    w.beta = reinterpret_cast<float*>(p); p = align(p + ng * 4);
    w.T = reinterpret_cast<_Float16*>(p); p = align(p + nm * 2);
    w.P = reinterpret_cast<_Float16*>(p);
    return w;
}

__device__ __forceinline__ f4 mma(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
__device__ __forceinline__ h8 ld8(const _Float16* p) { return *reinterpret_cast<const h8*>(p); }

// ------------------------------------------------------------ prep

struct alignas(16) PrepSmem {
    float yqk[CH / 2][2 * D];      // conv output of q|k for half a chunk (fp32, before the norm)
    _Float16 qh[CH][QKP];          // q^ (fp16)
    _Float16 kh[CH][QKP];          // k^ (fp16)
    float kk[CH][MP];              // K K^T (lower tiles)
    float qk[CH][MP];              // Q K^T (lower tiles)
    float A[CH][MP];               // A of one value head
    float T[CH][MP];               // its inverse (I + A)^-1
    float tmp[3][16][17];          // block products
    float G[MAXG][CH];
    float beta[MAXG][CH];
};

template <typename Act>
__global__ __launch_bounds__(256) void prep_kernel(const Act* __restrict__ x, const Act* __restrict__ tail,
                                                   const Act* __restrict__ w, const float* __restrict__ a,
                                                   const float* __restrict__ bg, Ws ws, int T, int seg0, int SP,
                                                   int nch, int Hk, int Hv, int C) {
    __shared__ PrepSmem sm;
    const int cl = blockIdx.x % nch;
    const int g = (blockIdx.x / nch) % Hk;
    const int bq = blockIdx.x / (nch * Hk);
    const int G = Hv / Hk;
    const int t_base = seg0 + cl * CH;           // first token of the chunk (prompt index)
    const int n = min(CH, T - t_base);           // valid tokens in the chunk
    const int s0 = cl * CH;                      // first token of the chunk (segment index)
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const size_t xrow = static_cast<size_t>(C);
    const Act* xb = x + static_cast<size_t>(bq) * T * xrow;
    const Act* tb = tail + static_cast<size_t>(bq) * C * 4;
    const int per_group = (2 + G) * D;

    for (int half = 0; half < 2; ++half) {
        // conv + SiLU: item = (channel of this group, 8 consecutive tokens)
        for (int item = threadIdx.x; item < per_group * 4; item += blockDim.x) {
            const int ch = item % per_group;
            const int tg = item / per_group;
            const int c = ch < D ? g * D + ch : ch < 2 * D ? Hk * D + g * D + (ch - D) : 2 * Hk * D + G * g * D + (ch - 2 * D);
            float wf[4];
            Quad<Act>::to_float(Quad<Act>::load(w + static_cast<size_t>(c) * 4), wf);
            const int tau0 = half * (CH / 2) + tg * 8;  // chunk-local token of the first output
            float hist[11];
#pragma unroll
            for (int m = 0; m < 11; ++m) {
                const int t = t_base + tau0 + m - 3;
                hist[m] = t < 0 ? widen(tb[static_cast<size_t>(c) * 4 + 4 + t])
                                : (t < T ? widen(xb[static_cast<size_t>(t) * xrow + c]) : 0.0f);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int tau = tau0 + j;
                const float yv = (tau < n) ? conv_silu(wf, &hist[j]) : 0.0f;
                if (ch < 2 * D) {
                    sm.yqk[tau - half * (CH / 2)][ch] = yv;
                } else {
                    const int h = G * g + (ch - 2 * D) / D;
                    const int d = (ch - 2 * D) % D;
                    ws.v[((static_cast<size_t>(bq) * Hv + h) * SP + s0 + tau) * D + d] = static_cast<_Float16>(yv);
                }
            }
        }
        __syncthreads();
        // L2 norm of each token's q and k (one wave per vector)
        for (int vec = wave; vec < CH; vec += 4) {
            const int tl = vec >> 1, which = vec & 1;
            const float e0 = sm.yqk[tl][which * D + lane];
            const float e1 = sm.yqk[tl][which * D + lane + kWave];
            float ss = __builtin_fmaf(e1, e1, e0 * e0);
            ss = group_sum<kWave>(ss);
            const float r = 1.0f / sqrtf(ss + kEps);
            const _Float16 h0 = static_cast<_Float16>(e0 * r), h1 = static_cast<_Float16>(e1 * r);
            const int tau = half * (CH / 2) + tl;
            _Float16* dst = which ? &sm.kh[tau][0] : &sm.qh[tau][0];
            dst[lane] = h0;
            dst[lane + kWave] = h1;
            _Float16* gdst = (which ? ws.k : ws.q) + ((static_cast<size_t>(bq) * Hk + g) * SP + s0 + tau) * D;
            gdst[lane] = h0;
            gdst[lane + kWave] = h1;
        }
        __syncthreads();
    }

    // gates: one wave per value head, one lane per token; inclusive scan of log alpha
    for (int hh = wave; hh < G; hh += 4) {
        const int h = G * g + hh;
        const bool valid = lane < n;
        float la = 0.0f, be = 0.0f;
        if (valid) {
            const size_t idx = (static_cast<size_t>(bq) * T + t_base + lane) * Hv + h;
            const float av = a[idx], bv = bg[idx];
            la = -(fmaxf(av, 0.0f) + log1pf(expf(-fabsf(av))));
            be = 1.0f / (1.0f + expf(-bv));
        }
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const float up = __shfl_up(la, off, kWave);
            if (lane >= off)
                la += up;
        }
        sm.G[hh][lane] = la;
        sm.beta[hh][lane] = be;
        const size_t gi = (static_cast<size_t>(bq) * Hv + h) * SP + s0 + lane;
        ws.G[gi] = la;
        ws.beta[gi] = be;
    }

    // K K^T and Q K^T, lower 16x16 tiles, on MFMA
    {
        constexpr int ti[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
        constexpr int tj[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
        for (int job = wave; job < 20; job += 4) {
            const int which = job / 10, I = ti[job % 10], J = tj[job % 10];
            const _Float16(*arow)[QKP] = which ? sm.qh : sm.kh;
            f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < D / 32; ++s)
                acc = mma(ld8(&arow[16 * I + (lane & 15)][32 * s + 8 * (lane >> 4)]),
                          ld8(&sm.kh[16 * J + (lane & 15)][32 * s + 8 * (lane >> 4)]), acc);
            float(*out)[MP] = which ? sm.qk : sm.kk;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                out[16 * I + 4 * (lane >> 4) + r][16 * J + (lane & 15)] = acc[r];
        }
        // k^ transposed per chunk, for the state update's B operand
        for (int item = threadIdx.x; item < D * (CH / 8); item += blockDim.x) {
            const int d = item / (CH / 8), oct = item % (CH / 8);
            h8 v;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                v[j] = sm.kh[8 * oct + j][d];
            *reinterpret_cast<h8*>(ws.kt + (((static_cast<size_t>(bq) * Hk + g) * (SP / CH) + cl) * D + d) * CH +
                                   8 * oct) = v;
        }
    }
    __syncthreads();

    const int nchp = SP / CH;
    for (int hh = 0; hh < G; ++hh) {
        const int h = G * g + hh;
        const size_t mbase = ((static_cast<size_t>(bq) * Hv + h) * nchp + cl) * CH * CH;
        for (int e = threadIdx.x; e < CH * CH; e += blockDim.x) {
            const int i = e / CH, j = e % CH;
            const float dg = (i >= j) ? expf(sm.G[hh][i] - sm.G[hh][j]) : 0.0f;
            sm.A[i][j] = (i > j) ? sm.beta[hh][i] * dg * sm.kk[i][j] : 0.0f;
            ws.P[mbase + e] = static_cast<_Float16>((i >= j) ? dg * sm.qk[i][j] : 0.0f);
        }
        __syncthreads();
        // diagonal 16x16 blocks of (I + A)^-1 by forward substitution, lane = column
        if (lane < 16) {
            const int o = 16 * wave, j = lane;
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
        // off-diagonal blocks, one block diagonal at a time:
        //   T_ij = -T_ii * sum_{k=j}^{i-1} A_ik T_kj
        for (int lvl = 1; lvl < 4; ++lvl) {
            const int nb = 4 - lvl;  // blocks on this diagonal: (lvl + q, q)
            for (int e = threadIdx.x; e < nb * 256; e += blockDim.x) {
                const int q = e / 256, r = (e / 16) % 16, c = e % 16;
                const int I = lvl + q, J = q;
                float s = 0.0f;
                for (int K = J; K < I; ++K)
                    for (int k = 0; k < 16; ++k)
                        s = __builtin_fmaf(sm.A[16 * I + r][16 * K + k], sm.T[16 * K + k][16 * J + c], s);
                sm.tmp[q][r][c] = s;
            }
            __syncthreads();
            for (int e = threadIdx.x; e < nb * 256; e += blockDim.x) {
                const int q = e / 256, r = (e / 16) % 16, c = e % 16;
                const int I = lvl + q, J = q;
                float s = 0.0f;
                for (int k = 0; k < 16; ++k)
                    s = __builtin_fmaf(sm.T[16 * I + r][16 * I + k], sm.tmp[q][k][c], s);
                sm.T[16 * I + r][16 * J + c] = -s;
            }
            __syncthreads();
        }
        for (int e = threadIdx.x; e < CH * CH; e += blockDim.x) {
            const int i = e / CH, j = e % CH;
            ws.T[mbase + e] = static_cast<_Float16>((j / 16 <= i / 16) ? sm.T[i][j] : 0.0f);
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ scan

struct alignas(16) ScanSmem {
    _Float16 s0[DS][QKP];   // S0 slice, fp16, [row][key]
    _Float16 rhsT[DS][CH + 8];
    _Float16 ut[DS][CH + 8];
    _Float16 utd[DS][CH + 8];
};

__global__ __launch_bounds__(256) void scan_kernel(float* __restrict__ S, float* __restrict__ o, Ws ws, int T,
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
    const int lr = lane & 15, lq = lane >> 4;
    const int nchp = SP / CH;

    float* Sh = S + ((static_cast<size_t>(bq) * Hv + h) * D + row0) * D;
    f4 sacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            sacc[tt][r] = Sh[(4 * lq + r) * D + 16 * (2 * wave + tt) + lr];

    const _Float16* qg = ws.q + (static_cast<size_t>(bq) * Hk + g) * SP * D;
    const _Float16* kg = ws.k + (static_cast<size_t>(bq) * Hk + g) * SP * D;
    const _Float16* ktg = ws.kt + (static_cast<size_t>(bq) * Hk + g) * nchp * D * CH;
    const _Float16* vh = ws.v + (static_cast<size_t>(bq) * Hv + h) * SP * D;
    const float* Gh = ws.G + (static_cast<size_t>(bq) * Hv + h) * SP;
    const float* bh = ws.beta + (static_cast<size_t>(bq) * Hv + h) * SP;
    const _Float16* Th = ws.T + (static_cast<size_t>(bq) * Hv + h) * nchp * CH * CH;
    const _Float16* Ph = ws.P + (static_cast<size_t>(bq) * Hv + h) * nchp * CH * CH;

    for (int cl = 0; cl < nch; ++cl) {
        const int t_base = seg0 + cl * CH;
        const int n = min(CH, T - t_base);
        const int s0 = cl * CH;
        const int trow = s0 + 16 * wave + lr;  // token row of this lane's A fragments
        h8 kf[4], qf[4], tf[2], pf[2], ktf[2][2];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            kf[s] = ld8(kg + static_cast<size_t>(trow) * D + 32 * s + 8 * lq);
            qf[s] = ld8(qg + static_cast<size_t>(trow) * D + 32 * s + 8 * lq);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            tf[s] = ld8(Th + (static_cast<size_t>(cl) * CH + 16 * wave + lr) * CH + 32 * s + 8 * lq);
            pf[s] = ld8(Ph + (static_cast<size_t>(cl) * CH + 16 * wave + lr) * CH + 32 * s + 8 * lq);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                ktf[tt][s] = ld8(ktg + (static_cast<size_t>(cl) * D + 16 * (2 * wave + tt) + lr) * CH + 32 * s + 8 * lq);
        }
        float vv[4], gv[4], bv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = s0 + 16 * wave + 4 * lq + r;
            vv[r] = static_cast<float>(vh[static_cast<size_t>(t) * D + row0 + lr]);
            gv[r] = Gh[t];
            bv[r] = bh[t];
        }
        const float glast = Gh[s0 + CH - 1];

        // S0 slice to LDS as fp16 [row][key]
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sm.s0[4 * lq + r][16 * (2 * wave + tt) + lr] = static_cast<_Float16>(sacc[tt][r]);
        __syncthreads();

        // X = K S0^T and Y = Q S0^T for tokens 16*wave .. +15
        f4 X = {0.0f, 0.0f, 0.0f, 0.0f}, Y = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const h8 bs = ld8(&sm.s0[lr][32 * s + 8 * lq]);
            X = mma(kf[s], bs, X);
            Y = mma(qf[s], bs, Y);
        }
        float eg[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            eg[r] = expf(gv[r]);
            const float rhs = bv[r] * (vv[r] - eg[r] * X[r]);
            sm.rhsT[lr][16 * wave + 4 * lq + r] = static_cast<_Float16>(rhs);
        }
        __syncthreads();

        // U = T rhs
        f4 U = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 2; ++s)
            U = mma(tf[s], ld8(&sm.rhsT[lr][32 * s + 8 * lq]), U);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * wave + 4 * lq + r;
            sm.ut[lr][t] = static_cast<_Float16>(U[r]);
            sm.utd[lr][t] = static_cast<_Float16>(U[r] * expf(glast - gv[r]));
        }
        __syncthreads();

        // O = s (e^G Y + P U)
        f4 PU = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 2; ++s)
            PU = mma(pf[s], ld8(&sm.ut[lr][32 * s + 8 * lq]), PU);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * wave + 4 * lq + r;
            if (t < n)
                o[((static_cast<size_t>(bq) * T + t_base + t) * Hv + h) * D + row0 + lr] =
                    kScale * __builtin_fmaf(eg[r], Y[r], PU[r]);
        }

        // S <- e^{G_n} S + U^T (e^{G_n - G} K)
        const float gl = expf(glast);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[tt][r] *= gl;
#pragma unroll
            for (int s = 0; s < 2; ++s)
                sacc[tt] = mma(ld8(&sm.utd[lr][32 * s + 8 * lq]), ktf[tt][s], sacc[tt]);
        }
    }

#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Sh[(4 * lq + r) * D + 16 * (2 * wave + tt) + lr] = sacc[tt][r];
}

// ------------------------------------------------------------ tail

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
    if (g.D != pf::D || g.Hv / g.Hk > pf::MAXG)
        return 0;
    return pf::ws_bytes(g.B, g.Hk, g.Hv, pf::seg_pitch(T));
}

hipError_t launch_prefill(const Geo& g, float* S, void* tail, const void* w, int T, const void* x, const float* a,
                          const float* b, float* o, void* ws, hipStream_t s) {
    if (g.D != pf::D || g.Hv / g.Hk > pf::MAXG)
        return hipErrorNotSupported;
    const size_t SP = pf::seg_pitch(T);
    const pf::Ws W = pf::carve(ws, g.B, g.Hk, g.Hv, SP);
    const int G = g.Hv / g.Hk;
    const int units = g.B * g.Hk;
    const int scan_grid = 8 * ((units + 7) / 8) * G * pf::NS;
    for (int seg0 = 0; seg0 < T; seg0 += pf::SEG) {
        const int len = std::min(pf::SEG, T - seg0);
        const int nch = (len + pf::CH - 1) / pf::CH;
        const dim3 pgrid(static_cast<unsigned>(g.B * g.Hk * nch)), block(256);
        if (g.bf16)
            hipLaunchKernelGGL(pf::prep_kernel<uint16_t>, pgrid, block, 0, s, static_cast<const uint16_t*>(x),
                               static_cast<const uint16_t*>(tail), static_cast<const uint16_t*>(w), a, b, W, T, seg0,
                               static_cast<int>(SP), nch, g.Hk, g.Hv, g.C);
        else
            hipLaunchKernelGGL(pf::prep_kernel<float>, pgrid, block, 0, s, static_cast<const float*>(x),
                               static_cast<const float*>(tail), static_cast<const float*>(w), a, b, W, T, seg0,
                               static_cast<int>(SP), nch, g.Hk, g.Hv, g.C);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(pf::scan_kernel, dim3(static_cast<unsigned>(scan_grid)), block, 0, s, S, o, W, T, seg0,
                           static_cast<int>(SP), nch, g.B, g.Hk, g.Hv);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const int64_t total = static_cast<int64_t>(g.B) * g.C;
    const dim3 tgrid(static_cast<unsigned>((total + 255) / 256)), block(256);
    if (g.bf16)
        hipLaunchKernelGGL(pf::tail_kernel<uint16_t>, tgrid, block, 0, s, static_cast<const uint16_t*>(x),
                           static_cast<uint16_t*>(tail), T, g.C, total);
    else
        hipLaunchKernelGGL(pf::tail_kernel<float>, tgrid, block, 0, s, static_cast<const float*>(x),
                           static_cast<float*>(tail), T, g.C, total);
    return hipGetLastError();
}

}  // namespace gdn
