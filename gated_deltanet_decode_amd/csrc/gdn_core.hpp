// gdn_core.hpp -- the per-token arithmetic shared by every recurrent kernel.
//
// Decode, tree verify and commit must agree bit for bit (the repository
// "Architecture" page says of the second model that its verify rows equal its
// decode rows bit for bit; section 8.1 of the first page asks for exact undo
// and branch).  Floating point does not associate, so the three kernels call
// the functions below and nothing else for: the conv tap sum and SiLU, the
// gates, the q/k L2 norm and k.q reduction (one fixed wave-wide butterfly),
// and the row update (one fixed lane-to-column map and butterfly).  The build
// passes -ffp-contract=off; every fused multiply-add here is written out.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr float kEps = 1e-6f;  // q/k L2-norm epsilon
constexpr int kWave = 64;
constexpr int kMaxNodes = 32;
constexpr int kMaxDepth = 8;

template <int D>
struct Scale;  // 1/sqrt(dk), written as the correctly rounded fp32 constant
template <>
struct Scale<32> { static constexpr float value = 0.17677669529663687f; };
template <>
struct Scale<128> { static constexpr float value = 0.08838834764831845f; };

// ------------------------------------------------------------ activation storage

// bf16 activations travel as raw 16-bit patterns; widening is a shift.
__device__ __forceinline__ float widen(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }
__device__ __forceinline__ float widen(float f) { return f; }

// Four consecutive activation values (one tail or weight row).
template <typename Act>
struct Quad;
template <>
struct Quad<uint16_t> {
    using raw = uint2;
    __device__ static raw load(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }
    __device__ static void store(uint16_t* p, raw v) { *reinterpret_cast<uint2*>(p) = v; }
    __device__ static void to_float(raw v, float f[4]) {
        f[0] = __uint_as_float(v.x << 16);
        f[1] = __uint_as_float(v.x & 0xFFFF0000u);
        f[2] = __uint_as_float(v.y << 16);
        f[3] = __uint_as_float(v.y & 0xFFFF0000u);
    }
    // shift left by one element and append `in` (raw bits)
    __device__ static raw push(raw v, uint16_t in) {
        raw r;
        r.x = (v.x >> 16) | (v.y << 16);
        r.y = (v.y >> 16) | (static_cast<uint32_t>(in) << 16);
        return r;
    }
    __device__ static uint16_t elem(raw v, int j) {
        uint32_t w = (j < 2) ? v.x : v.y;
        return static_cast<uint16_t>((j & 1) ? (w >> 16) : (w & 0xFFFFu));
    }
};
template <>
struct Quad<float> {
    using raw = float4;
    __device__ static raw load(const float* p) { return *reinterpret_cast<const float4*>(p); }
    __device__ static void store(float* p, raw v) { *reinterpret_cast<float4*>(p) = v; }
    __device__ static void to_float(raw v, float f[4]) { f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w; }
    __device__ static raw push(raw v, float in) { return make_float4(v.y, v.z, v.w, in); }
    __device__ static float elem(raw v, int j) { return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w; }
};

// State rows are streamed once per call: non-temporal loads and stores keep
// them from displacing what the caches hold for reuse.
typedef float nt4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream(const float* p) {
    const nt4 v = __builtin_nontemporal_load(reinterpret_cast<const nt4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(float* p, float4 v) {
    __builtin_nontemporal_store(nt4{v.x, v.y, v.z, v.w}, reinterpret_cast<nt4*>(p));
}

// ------------------------------------------------------------ scalar pieces

// y = SiLU(sum_j w[j] * win[j]) with the taps summed oldest first.  SiLU(z)
// = z / (1 + e^-z) with e^-z = 2^(-z log2 e) and the reciprocal both on the
// hardware (about one ulp each): 9 instructions against 31 for the libm exp
// and an IEEE divide, which matters where every channel of every node is
// convolved.  Every call that convolves uses this one function, so decode,
// verify and commit still agree bit for bit.
__device__ __forceinline__ float conv_silu(const float w[4], const float win[4]) {
    float acc = w[0] * win[0];
    acc = __builtin_fmaf(w[1], win[1], acc);
    acc = __builtin_fmaf(w[2], win[2], acc);
    acc = __builtin_fmaf(w[3], win[3], acc);
    return acc * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(acc * -1.4426950408889634f));
}

// alpha = exp(-softplus(a)) = 1 / (1 + e^a);  beta = sigmoid(b) = 1 / (1 + e^-b).
__device__ __forceinline__ float forget_gate(float a) { return 1.0f / (1.0f + expf(a)); }
__device__ __forceinline__ float write_gate(float b) { return 1.0f / (1.0f + expf(-b)); }
__device__ __forceinline__ void gates(float a, float b, float& alpha, float& beta) {
    alpha = forget_gate(a);
    beta = write_gate(b);
}

// ------------------------------------------------------------ wave reductions

// Sum over aligned groups of `Width` lanes (4, 8, 16 or 64) with DPP lane
// moves, which read a neighbour's register without going through LDS:
//   xor 1 and xor 2 inside a quad, then the half-row mirror (quad q with quad
//   q^1), then the row mirror (the two halves of a 16-lane row).
// Each step adds two numbers that the partner lane adds in the other order,
// so every lane of a group ends with the same bits.  For 64 lanes the four row
// sums are read into scalar registers and added in a fixed order.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int Width>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(Width == 4 || Width == 8 || Width == 16 || Width == 64, "unsupported group width");
    v += dpp_move<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_move<0x4E>(v);   // quad_perm [2,3,0,1]
    if constexpr (Width >= 8)
        v += dpp_move<0x141>(v);  // row_half_mirror
    if constexpr (Width >= 16)
        v += dpp_move<0x140>(v);  // row_mirror
    if constexpr (Width == 64) {
        const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
        const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
        const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
        const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
        v = (r0 + r1) + (r2 + r3);
    }
    return v;
}

// ------------------------------------------------------------ q/k preparation

// One wave normalises one token's q~ and k~ of one q/k head.  Lane l holds
// elements l + 64*j (j < J); lanes past D hold zeros.  On return they hold q^,
// k^ and every lane holds kq = k^.q^.  The three sums (|q~|^2, |k~|^2, q~.k~)
// are reduced together, and kq is formed from q~.k~ and the two reciprocal
// norms, so one wave reduction stands between the conv outputs and the row
// update instead of two.
template <int D>
struct Prep {
    static constexpr int J = D >= kWave ? D / kWave : 1;
};

template <int D>
__device__ __forceinline__ void prep_qk(float (&q)[Prep<D>::J], float (&k)[Prep<D>::J], float& kq) {
    constexpr int J = Prep<D>::J;
    float nq = 0.0f, nk = 0.0f, d = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        nq = __builtin_fmaf(q[j], q[j], nq);
        nk = __builtin_fmaf(k[j], k[j], nk);
        d = __builtin_fmaf(q[j], k[j], d);
    }
    nq = group_sum<kWave>(nq);
    nk = group_sum<kWave>(nk);
    d = group_sum<kWave>(d);
    const float rq = __builtin_amdgcn_rsqf(nq + kEps);   // hardware reciprocal square root, about 1 ulp
    const float rk = __builtin_amdgcn_rsqf(nk + kEps);
#pragma unroll
    for (int j = 0; j < J; ++j) {
        q[j] = q[j] * rq;
        k[j] = k[j] * rk;
    }
    kq = d * rq * rk;
}

// ------------------------------------------------------------ the row update

// A state row of D keys is spread over LPR consecutive lanes; lane r of the
// group holds the float4 vectors at keys j*4*LPR + 4*r .. +3 for j < NV.
template <int D>
struct Row {
    static constexpr int LPR = (D == 128) ? 16 : 8;
    static constexpr int NV = D / (4 * LPR);
    static constexpr int RPW = kWave / LPR;  // rows per wave
    __device__ static int key(int j, int r) { return j * 4 * LPR + 4 * r; }
};

__device__ __forceinline__ float dot4(float4 s, float4 k, float acc) {
    acc = __builtin_fmaf(s.x, k.x, acc);
    acc = __builtin_fmaf(s.y, k.y, acc);
    acc = __builtin_fmaf(s.z, k.z, acc);
    acc = __builtin_fmaf(s.w, k.w, acc);
    return acc;
}

__device__ __forceinline__ float4 axpby4(float u, float4 k, float alpha, float4 s) {
    return make_float4(__builtin_fmaf(u, k.x, alpha * s.x), __builtin_fmaf(u, k.y, alpha * s.y),
                       __builtin_fmaf(u, k.z, alpha * s.z), __builtin_fmaf(u, k.w, alpha * s.w));
}

// One token on one row S[i,:] (this lane's slice in s):
//   p = alpha (S.k);  u = beta (v_i - p);  S <- alpha S + u k;
//   o_i = scale (alpha (S_old.q) + u (k.q))   [= scale (S_new.q)]
// Both dot products come from one pass over the old row.  Returns o_i on every
// lane of the row group.
template <int D>
__device__ __forceinline__ float row_update(float4 (&s)[Row<D>::NV], const float4 (&k)[Row<D>::NV],
                                            const float4 (&q)[Row<D>::NV], float alpha, float beta,
                                            float v, float kq) {
    constexpr int NV = Row<D>::NV;
    float pk = 0.0f, pq = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        pk = dot4(s[j], k[j], pk);
        pq = dot4(s[j], q[j], pq);
    }
    pk = group_sum<Row<D>::LPR>(pk);
    pq = group_sum<Row<D>::LPR>(pq);
    const float u = beta * (v - alpha * pk);
#pragma unroll
    for (int j = 0; j < NV; ++j)
        s[j] = axpby4(u, k[j], alpha, s[j]);
    return Scale<D>::value * __builtin_fmaf(u, kq, alpha * pq);
}

// The per-channel-decay step on one row: the forget gate is a vector over the
// key channels, applied to the row before the delta correction:
//   S' = S diag(al);  u = beta (v_i - S'.k);  S <- S' + u k;  o_i = scale (S'.q + u (k.q))
// ka = al * k and qa = al * q (elementwise, shared by every row of the head)
// give both dot products of S' from one pass over the old row.
template <int D>
__device__ __forceinline__ float row_update_kda(float4 (&s)[Row<D>::NV], const float4 (&k)[Row<D>::NV],
                                                const float4 (&ka)[Row<D>::NV], const float4 (&qa)[Row<D>::NV],
                                                const float4 (&al)[Row<D>::NV], float beta, float v, float kq) {
    constexpr int NV = Row<D>::NV;
    float pk = 0.0f, pq = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        pk = dot4(s[j], ka[j], pk);
        pq = dot4(s[j], qa[j], pq);
    }
    pk = group_sum<Row<D>::LPR>(pk);
    pq = group_sum<Row<D>::LPR>(pq);
    const float u = beta * (v - pk);
#pragma unroll
    for (int j = 0; j < NV; ++j)
        s[j] = make_float4(__builtin_fmaf(u, k[j].x, al[j].x * s[j].x), __builtin_fmaf(u, k[j].y, al[j].y * s[j].y),
                           __builtin_fmaf(u, k[j].z, al[j].z * s[j].z), __builtin_fmaf(u, k[j].w, al[j].w * s[j].w));
    return Scale<D>::value * __builtin_fmaf(u, kq, pq);
}

// Forget gates of this lane's keys from their gate inputs (laid out as k):
// alpha = 1 / (1 + e^a) with e^a = 2^(a log2 e) and the reciprocal on the
// hardware (about one ulp each, as in conv_silu), since every lane forms
// 4 * NV of them on the way to its first row update.  e^a overflowing gives
// alpha = 0, and underflowing gives alpha = 1, the limits of the gate.
__device__ __forceinline__ float forget_gate_hw(float a) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a * 1.4426950408889634f));
}

template <int D>
__device__ __forceinline__ void kda_gates(const float4 (&araw)[Row<D>::NV], float4 (&al)[Row<D>::NV]) {
#pragma unroll
    for (int j = 0; j < Row<D>::NV; ++j)
        al[j] = make_float4(forget_gate_hw(araw[j].x), forget_gate_hw(araw[j].y), forget_gate_hw(araw[j].z),
                            forget_gate_hw(araw[j].w));
}

// The gated key and query vectors row_update_kda takes: ka = al * k, qa = al * q.
template <int D>
__device__ __forceinline__ void kda_vectors(const float4 (&al)[Row<D>::NV], const float4 (&k)[Row<D>::NV],
                                            const float4 (&q)[Row<D>::NV], float4 (&ka)[Row<D>::NV],
                                            float4 (&qa)[Row<D>::NV]) {
#pragma unroll
    for (int j = 0; j < Row<D>::NV; ++j) {
        ka[j] = make_float4(al[j].x * k[j].x, al[j].y * k[j].y, al[j].z * k[j].z, al[j].w * k[j].w);
        qa[j] = make_float4(al[j].x * q[j].x, al[j].y * q[j].y, al[j].z * q[j].z, al[j].w * q[j].w);
    }
}

}  // namespace gdn
