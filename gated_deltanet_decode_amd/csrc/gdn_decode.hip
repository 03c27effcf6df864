// gdn_decode.hip -- one token: the conv update and the state step.
//
// The state step streams each sequence's Hv x dv x dk fp32 state through
// registers once, reading and writing every element exactly once (section 8.1
// of the "Architecture" page: 48 heads of 128 x 128 fp32 per layer, updated
// per token; the CPU page: a rank-1 update written in place).  It is bound by
// HBM bandwidth: ~6.3 MB of state traffic per sequence-token against a few
// KB of vectors.  Layout per workgroup: one (sequence, value head) and a block
// of rows; 4 waves; a row's 128 keys sit on 16 lanes as two float4 each, so
// every wave-wide load is four fully used 256-byte row segments.  The state
// loads are issued before anything else so their latency overlaps the q/k
// normalisation, which one wave does into LDS.
#include "gdn_core.hpp"
#include "gdn_launch.hpp"

namespace gdn {

// ------------------------------------------------------------ conv update

template <typename Act>
__global__ __launch_bounds__(256) void conv_update_kernel(const Act* __restrict__ x, Act* __restrict__ tail,
                                                          const Act* __restrict__ w, float* __restrict__ y, int C,
                                                          int64_t total) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= total)
        return;
    const int c = static_cast<int>(i % C);
    using Q = Quad<Act>;
    const typename Q::raw t = Q::push(Q::load(tail + i * 4), x[i]);
    Q::store(tail + i * 4, t);
    float win[4], wf[4];
    Q::to_float(t, win);
    Q::to_float(Q::load(w + static_cast<int64_t>(c) * 4), wf);
    y[i] = conv_silu(wf, win);
}

hipError_t launch_conv_update(const Geo& g, const void* x, void* tail, const void* w, float* y, hipStream_t s) {
    const int64_t total = static_cast<int64_t>(g.B) * g.C;
    const dim3 block(256), grid(static_cast<unsigned>((total + 255) / 256));
    if (g.bf16)
        hipLaunchKernelGGL(conv_update_kernel<uint16_t>, grid, block, 0, s, static_cast<const uint16_t*>(x),
                           static_cast<uint16_t*>(tail), static_cast<const uint16_t*>(w), y, g.C, total);
    else
        hipLaunchKernelGGL(conv_update_kernel<float>, grid, block, 0, s, static_cast<const float*>(x),
                           static_cast<float*>(tail), static_cast<const float*>(w), y, g.C, total);
    return hipGetLastError();
}

// ------------------------------------------------------------ state step

// PASSES row-quads per wave; a workgroup covers 4 * RPW * PASSES rows of one head.
// KDA: the forget gate is per key channel, a is [B][Hv][D] (row_update_kda).
template <int D, int PASSES, bool KDA>
__global__ __launch_bounds__(256) void decode_kernel(float* __restrict__ S, const float* __restrict__ y,
                                                     const float* __restrict__ a, const float* __restrict__ b,
                                                     float* __restrict__ o, int Hk, int Hv, int C,
                                                     int blocks_per_head) {
    using R = Row<D>;
    constexpr int NV = R::NV, LPR = R::LPR, RPW = R::RPW;
    constexpr int ROWS_PASS = 4 * RPW;
    constexpr int J = Prep<D>::J;

    // The index arithmetic is made to depend on every argument, so all the
    // argument loads issue together (one kernel-argument round trip).
    asm volatile("" : "+s"(blocks_per_head) : "s"(S), "s"(y), "s"(a), "s"(b), "s"(o), "s"(Hk), "s"(Hv), "s"(C));
    const int blk = blockIdx.x % blocks_per_head;
    const int bh = blockIdx.x / blocks_per_head;  // sequence * Hv + head
    const int h = bh % Hv;
    const int seq = bh / Hv;
    const int grp = h / (Hv / Hk);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r = lane % LPR;

    // The per-channel gate inputs go before the state loads, so their gates are
    // computed while the state is in flight.
    float4 al[NV];
    if constexpr (KDA) {
        float4 araw[NV];
#pragma unroll
        for (int j = 0; j < NV; ++j)
            araw[j] = *reinterpret_cast<const float4*>(a + static_cast<size_t>(bh) * D + R::key(j, r));
        kda_gates<D>(araw, al);
    }
    float* Sh = S + static_cast<size_t>(bh) * D * D;
    int row[PASSES];
    float4 s[PASSES][NV];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        row[p] = (blk * PASSES + p) * ROWS_PASS + wave * RPW + lane / LPR;
#pragma unroll
        for (int j = 0; j < NV; ++j)
            s[p][j] = load_stream(Sh + row[p] * D + R::key(j, r));
    }

    __shared__ __align__(16) float qs[D];
    __shared__ __align__(16) float ks[D];
    __shared__ float kq_s;
    const float* ys = y + static_cast<size_t>(seq) * C;
    if (wave == 0) {
        float qv[J], kv[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int e = lane + kWave * j;
            qv[j] = e < D ? ys[grp * D + e] : 0.0f;
            kv[j] = e < D ? ys[Hk * D + grp * D + e] : 0.0f;
        }
        float kq;
        prep_qk<D>(qv, kv, kq);
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int e = lane + kWave * j;
            if (e < D) {
                qs[e] = qv[j];
                ks[e] = kv[j];
            }
        }
        if (lane == 0)
            kq_s = kq;
    }
    float alpha = 0.0f, beta;
    if constexpr (KDA)
        beta = write_gate(b[bh]);
    else
        gates(a[bh], b[bh], alpha, beta);
    float v[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
        v[p] = ys[2 * Hk * D + h * D + row[p]];
    __syncthreads();

    float4 kk[NV], qq[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        kk[j] = *reinterpret_cast<const float4*>(ks + R::key(j, r));
        qq[j] = *reinterpret_cast<const float4*>(qs + R::key(j, r));
    }
    const float kq = kq_s;
    float4 ka[NV], qa[NV];
    if constexpr (KDA)
        kda_vectors<D>(al, kk, qq, ka, qa);
    float* oh = o + static_cast<size_t>(bh) * D;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        float out;
        if constexpr (KDA)
            out = row_update_kda<D>(s[p], kk, ka, qa, al, beta, v[p], kq);
        else
            out = row_update<D>(s[p], kk, qq, alpha, beta, v[p], kq);
#pragma unroll
        for (int j = 0; j < NV; ++j)
            store_stream(Sh + row[p] * D + R::key(j, r), s[p][j]);
        if (r == 0)
            oh[row[p]] = out;
    }
}

template <int D, int PASSES, bool KDA>
static hipError_t launch_decode_cfg(const Geo& g, float* S, const float* y, const float* a, const float* b, float* o,
                                    hipStream_t s) {
    constexpr int ROWS_WG = 4 * Row<D>::RPW * PASSES;
    static_assert(D % ROWS_WG == 0, "rows per workgroup must divide the head");
    const int bph = D / ROWS_WG;
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(g.B) * g.Hv * bph)), block(256);
    hipLaunchKernelGGL((decode_kernel<D, PASSES, KDA>), grid, block, 0, s, S, y, a, b, o, g.Hk, g.Hv, g.C, bph);
    return hipGetLastError();
}

template <bool KDA>
static hipError_t launch_decode_kind(const Geo& g, float* S, const float* y, const float* a, const float* b,
                                     float* o, hipStream_t s) {
    if (g.D == 128) {
        // Few heads in flight (small batch): one row-quad per wave for the most waves.
        if (static_cast<int64_t>(g.B) * g.Hv < 512)
            return launch_decode_cfg<128, 1, KDA>(g, S, y, a, b, o, s);
        return launch_decode_cfg<128, 2, KDA>(g, S, y, a, b, o, s);
    }
    return launch_decode_cfg<32, 1, KDA>(g, S, y, a, b, o, s);
}

hipError_t launch_decode(const Geo& g, float* S, const float* y, const float* a, const float* b, float* o,
                         hipStream_t s) {
    return launch_decode_kind<false>(g, S, y, a, b, o, s);
}

hipError_t launch_kda_decode(const Geo& g, float* S, const float* y, const float* a, const float* b, float* o,
                             hipStream_t s) {
    return launch_decode_kind<true>(g, S, y, a, b, o, s);
}

}  // namespace gdn
