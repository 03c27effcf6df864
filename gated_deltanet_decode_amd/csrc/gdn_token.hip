// gdn_token.hip -- one whole token in one launch: conv update, q/k norm, gates
// and the state step ("Architecture" section 8.1: a fixed-size state and a
// 4-wide convolution tail advanced per token; CPU page: the state updated in
// place by a rank-1 product, the convolutions kept as rings of recent inputs).
//
// Same arithmetic, bit for bit, as gdn_conv_update followed by
// gdn_decode_step (both go through gdn_core.hpp), without the round trip of y
// through memory and without a second launch.  Every workgroup computes the
// conv outputs it needs itself: the 2*dk q/k channels of its q/k head (shared
// by the workgroups of that head's value heads) and the v channels of its own
// rows.  Because several workgroups read a q/k channel's window, the tail is
// updated out of place: all reads come from tail_in, and each channel of
// tail_out is written by exactly one workgroup (the v channels by the owner of
// their rows, a q/k head's channels by block 0 of its first value head).
//
// Load order matters on gfx9, whose memory counter retires in order: the few
// conv loads are issued first and the state loads after them, so waiting for
// the conv inputs does not wait for the state.
#include "gdn_core.hpp"
#include "gdn_launch.hpp"

namespace gdn {

// KDA: the forget gate is per key channel, a is [B][Hv][D] (row_update_kda).
template <int D, int PASSES, typename Act, bool KDA>
__global__ __launch_bounds__(256) void token_kernel(float* __restrict__ S, const Act* __restrict__ tail_in,
                                                    Act* __restrict__ tail_out, const Act* __restrict__ w,
                                                    const Act* __restrict__ x, const float* __restrict__ a,
                                                    const float* __restrict__ b, float* __restrict__ o, int Hk,
                                                    int Hv, int C, int blocks_per_head) {
    using R = Row<D>;
    using Q = Quad<Act>;
    constexpr int NV = R::NV, LPR = R::LPR, RPW = R::RPW;
    constexpr int ROWS_PASS = 4 * RPW;
    constexpr int ROWS_WG = ROWS_PASS * PASSES;
    constexpr int NCH = 2 * D + ROWS_WG;             // channels this workgroup convolves
    constexpr int SLOTS = (NCH + 255) / 256;         // channels per thread
    constexpr int J = Prep<D>::J;

    // The index arithmetic is made to depend on every argument, so all the
    // argument loads issue together and the input loads wait for one
    // kernel-argument round trip, not two.
    int bph = blocks_per_head;
    asm volatile("" : "+s"(bph) : "s"(S), "s"(tail_in), "s"(tail_out), "s"(w), "s"(x), "s"(a), "s"(b), "s"(o),
                 "s"(Hk), "s"(Hv), "s"(C));
    const int blk = blockIdx.x % bph;
    const int bh = blockIdx.x / bph;  // sequence * Hv + head
    const int h = bh % Hv;
    const int seq = bh / Hv;
    const int G = Hv / Hk;
    const int grp = h / G;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int r = lane % LPR;
    const int row_base = blk * ROWS_WG;
    const bool qk_writer = (h % G == 0) && blk == 0;

    // conv inputs first: channel ch of this workgroup's list -> global channel
    const Act* xs = x + static_cast<size_t>(seq) * C;
    const Act* ts = tail_in + static_cast<size_t>(seq) * C * 4;
    Act* tso = tail_out + static_cast<size_t>(seq) * C * 4;
    int chan[SLOTS];
    typename Q::raw traw[SLOTS], wraw[SLOTS];
    Act xin[SLOTS];
#pragma unroll
    for (int k = 0; k < SLOTS; ++k) {
        const int ch0 = tid + 256 * k;
        const int ch = ch0 < NCH ? ch0 : NCH - 1;   // clamped: loads stay unconditional
        chan[k] = ch < D ? grp * D + ch
                : ch < 2 * D ? Hk * D + grp * D + (ch - D)
                             : 2 * Hk * D + h * D + row_base + (ch - 2 * D);
        traw[k] = Q::load(ts + static_cast<size_t>(chan[k]) * 4);
        xin[k] = xs[chan[k]];
        wraw[k] = Q::load(w + static_cast<size_t>(chan[k]) * 4);
    }

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

    // then the state rows
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

    __shared__ __align__(16) float ys[NCH];
    __shared__ __align__(16) float qs[D];
    __shared__ __align__(16) float ks[D];
    __shared__ float kq_s;
#pragma unroll
    for (int k = 0; k < SLOTS; ++k) {
        const int ch0 = tid + 256 * k;
        const typename Q::raw t = Q::push(traw[k], xin[k]);
        if (ch0 < NCH && (ch0 >= 2 * D || qk_writer))
            Q::store(tso + static_cast<size_t>(chan[k]) * 4, t);
        float win[4], wf[4];
        Q::to_float(t, win);
        Q::to_float(wraw[k], wf);
        if (ch0 < NCH)
            ys[ch0] = conv_silu(wf, win);
    }
    __syncthreads();

    if (wave == 0) {
        float qv[J], kv[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int e = lane + kWave * j;
            qv[j] = e < D ? ys[e] : 0.0f;
            kv[j] = e < D ? ys[D + e] : 0.0f;
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
        const float v = ys[2 * D + row[p] - row_base];
        float out;
        if constexpr (KDA)
            out = row_update_kda<D>(s[p], kk, ka, qa, al, beta, v, kq);
        else
            out = row_update<D>(s[p], kk, qq, alpha, beta, v, kq);
#pragma unroll
        for (int j = 0; j < NV; ++j)
            store_stream(Sh + row[p] * D + R::key(j, r), s[p][j]);
        if (r == 0)
            oh[row[p]] = out;
    }
}

template <int D, int PASSES, typename Act, bool KDA>
static hipError_t launch_token_cfg(const Geo& g, float* S, const void* tail_in, void* tail_out, const void* w,
                                   const void* x, const float* a, const float* b, float* o, hipStream_t s) {
    constexpr int ROWS_WG = 4 * Row<D>::RPW * PASSES;
    const int bph = D / ROWS_WG;
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(g.B) * g.Hv * bph)), block(256);
    hipLaunchKernelGGL((token_kernel<D, PASSES, Act, KDA>), grid, block, 0, s, S, static_cast<const Act*>(tail_in),
                       static_cast<Act*>(tail_out), static_cast<const Act*>(w), static_cast<const Act*>(x), a, b, o,
                       g.Hk, g.Hv, g.C, bph);
    return hipGetLastError();
}

template <typename Act, bool KDA>
static hipError_t launch_token_act(const Geo& g, float* S, const void* tail_in, void* tail_out, const void* w,
                                   const void* x, const float* a, const float* b, float* o, hipStream_t s) {
    // Same geometry rule as the state step alone: two row-quads per wave once
    // there are enough (sequence, head) pairs to fill the chip.
    if (g.D == 128) {
        if (static_cast<int64_t>(g.B) * g.Hv < 512)
            return launch_token_cfg<128, 1, Act, KDA>(g, S, tail_in, tail_out, w, x, a, b, o, s);
        return launch_token_cfg<128, 2, Act, KDA>(g, S, tail_in, tail_out, w, x, a, b, o, s);
    }
    return launch_token_cfg<32, 1, Act, KDA>(g, S, tail_in, tail_out, w, x, a, b, o, s);
}

hipError_t launch_token(const Geo& g, float* S, const void* tail_in, void* tail_out, const void* w, const void* x,
                        const float* a, const float* b, float* o, hipStream_t s) {
    if (g.bf16)
        return launch_token_act<uint16_t, false>(g, S, tail_in, tail_out, w, x, a, b, o, s);
    return launch_token_act<float, false>(g, S, tail_in, tail_out, w, x, a, b, o, s);
}

hipError_t launch_kda_token(const Geo& g, float* S, const void* tail_in, void* tail_out, const void* w,
                            const void* x, const float* a, const float* b, float* o, hipStream_t s) {
    if (g.bf16)
        return launch_token_act<uint16_t, true>(g, S, tail_in, tail_out, w, x, a, b, o, s);
    return launch_token_act<float, true>(g, S, tail_in, tail_out, w, x, a, b, o, s);
}

}  // namespace gdn
