// gdn_selfcheck.hip -- the load-time self-check that gates speculation
// (repository "Architecture" page, "Kernels and devices, then the mesh": an
// exact model serves plain decode until its kernels are row-invariant, and a
// self-check at load time decides whether speculation may run).  For this
// mixer the property is that a tree verify's row for a node equals, bit for
// bit, the row that token-by-token decode produces at the end of the node's
// path, and that committing a path leaves the state decode leaves.
//
// On one seeded case of the caller's layer shape, generated on the device:
//   1. a 32-node tree (a chain of 8 from the root, the other 24 nodes hung
//      under its first seven) is verified by the exact walk, one launch;
//   2. 32 sequences, each a copy of the checkpoint, replay the root-first
//      paths to the 32 nodes with the fused decode call, 8 steps (a path
//      shorter than 8 repeats its last token; only the row at its end is
//      compared);
//   3. the path to the depth-8 node is committed from the checkpoint;
//   4. every output row of step 1 is compared bitwise with its decode row,
//      and the committed state and tail with decode's after 8 steps.
// The verdict goes to a device word; nothing is synchronised.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn.h"
#include "gdn_launch.hpp"

namespace gdn {
namespace sc {

constexpr int N = 32;      // tree nodes
constexpr int L = 8;       // replay steps = the deepest path
constexpr int CHAIN = 8;   // nodes 0..7 form a chain; node 7 is at depth 8

// Counter-based draws: a 32-bit integer hash of (seed, tensor, index), and
// roughly N(0, 1) values as the scaled sum of four uniform draws.
__device__ __forceinline__ uint32_t mix(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}
__device__ __forceinline__ float normalish(uint32_t seed, uint32_t tensor, uint32_t i) {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        s += static_cast<float>(mix(seed ^ mix(tensor * 0x9E3779B9u + 4 * i + j)) >> 8) * (1.0f / 16777216.0f);
    return (s - 2.0f) * 1.7320508f;
}
__device__ __forceinline__ uint16_t to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__host__ __device__ constexpr int parent_of(int i) { return i == 0 ? -1 : i < CHAIN ? i - 1 : (5 * i) % (CHAIN - 1); }

struct Ws {
    float *ckpt, *commit_S, *states;   // [Hv][D][D], [Hv][D][D], [N][Hv][D][D]
    void *ckpt_tail, *commit_tail, *tails0, *tails1, *w, *x_nodes, *x_steps;
    float *a_nodes, *b_nodes, *a_steps, *b_steps;   // [N][Hv], [L][N][Hv]
    float *o_tree, *o_steps;                        // [N][Hv][D], [L][N][Hv][D]
    int32_t *parent, *path, *status;                // [N], [L], [4]: tree, commit, unused, unused
    void* tree_ws;
};

inline size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

inline size_t carve(const Geo& g, void* base, Ws* w) {
    const size_t es = g.bf16 ? 2 : 4;
    const size_t sb = static_cast<size_t>(g.Hv) * g.D * g.D * 4, tb = static_cast<size_t>(g.C) * 4 * es;
    const size_t xb = static_cast<size_t>(g.C) * es, gb = static_cast<size_t>(g.Hv) * 4;
    const size_t ob = static_cast<size_t>(g.Hv) * g.D * 4;
    uintptr_t p = align256(reinterpret_cast<uintptr_t>(base));
    const uintptr_t p0 = p;
    auto take = [&](size_t n) { void* r = reinterpret_cast<void*>(p); p += align256(n); return r; };
    Ws v;
    v.ckpt = static_cast<float*>(take(sb));
    v.commit_S = static_cast<float*>(take(sb));
    v.states = static_cast<float*>(take(sb * N));
    v.ckpt_tail = take(tb);
    v.commit_tail = take(tb);
    v.tails0 = take(tb * N);
    v.tails1 = take(tb * N);
    v.w = take(tb);
    v.x_nodes = take(xb * N);
    v.x_steps = take(xb * N * L);
    v.a_nodes = static_cast<float*>(take(gb * N));
    v.b_nodes = static_cast<float*>(take(gb * N));
    v.a_steps = static_cast<float*>(take(gb * N * L));
    v.b_steps = static_cast<float*>(take(gb * N * L));
    v.o_tree = static_cast<float*>(take(ob * N));
    v.o_steps = static_cast<float*>(take(ob * N * L));
    v.parent = static_cast<int32_t*>(take(N * 4));
    v.path = static_cast<int32_t*>(take(L * 4));
    v.status = static_cast<int32_t*>(take(4 * 4));
    v.tree_ws = take(tree_ws_bytes(1, N, g.Hk, g.Hv, g.D));
    if (w)
        *w = v;
    return (p - p0) + 256;   // + the worst-case alignment of base
}

// Fills the case: checkpoint state ~ 0.1 N, tail and x ~ N, weights ~ 0.5 N,
// gates ~ N; the tree, the path to node 7, and zeroes the verdict.
template <typename Act>
__global__ __launch_bounds__(256) void gen_kernel(Ws w, int Hv, int D, int C, uint32_t seed, int32_t* result) {
    const size_t nS = static_cast<size_t>(Hv) * D * D;
    const size_t nT = static_cast<size_t>(C) * 4;
    const size_t nX = static_cast<size_t>(C) * N;
    const size_t nG = static_cast<size_t>(Hv) * N;
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    const size_t i0 = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    auto act = [](float f) -> Act {
        if constexpr (sizeof(Act) == 2)
            return to_bf16(f);
        else
            return f;
    };
    for (size_t i = i0; i < nS; i += stride)
        w.ckpt[i] = 0.1f * normalish(seed, 1, static_cast<uint32_t>(i));
    for (size_t i = i0; i < nT; i += stride) {
        static_cast<Act*>(w.ckpt_tail)[i] = act(normalish(seed, 2, static_cast<uint32_t>(i)));
        static_cast<Act*>(w.w)[i] = act(0.5f * normalish(seed, 3, static_cast<uint32_t>(i)));
    }
    for (size_t i = i0; i < nX; i += stride)
        static_cast<Act*>(w.x_nodes)[i] = act(normalish(seed, 4, static_cast<uint32_t>(i)));
    for (size_t i = i0; i < nG; i += stride) {
        w.a_nodes[i] = normalish(seed, 5, static_cast<uint32_t>(i));
        w.b_nodes[i] = normalish(seed, 6, static_cast<uint32_t>(i));
    }
    if (i0 < N)
        w.parent[i0] = parent_of(static_cast<int>(i0));
    if (i0 < L)
        w.path[i0] = static_cast<int32_t>(i0);
    if (i0 < 4) {
        w.status[i0] = -1;
        result[i0] = 0;
    }
}

// Per replay sequence n and step j, the token of its root-first path (the
// last one again once the path has ended), optionally flipped in one input
// bit for sequence N-1; the 32 decode states and tails and the commit's state
// and tail start as copies of the checkpoint.
template <typename Act>
__global__ __launch_bounds__(256) void expand_kernel(Ws w, int Hv, int D, int C, int perturb) {
    const size_t nS = static_cast<size_t>(Hv) * D * D;
    const size_t nT = static_cast<size_t>(C) * 4;
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    const size_t i0 = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    for (size_t i = i0; i < nS; i += stride) {
        const float v = w.ckpt[i];
        w.commit_S[i] = v;
        for (int n = 0; n < N; ++n)
            w.states[n * nS + i] = v;
    }
    for (size_t i = i0; i < nT; i += stride) {
        const Act v = static_cast<const Act*>(w.ckpt_tail)[i];
        static_cast<Act*>(w.commit_tail)[i] = v;
        for (int n = 0; n < N; ++n)
            static_cast<Act*>(w.tails0)[n * nT + i] = v;
    }
    // (step, sequence) pairs: one per workgroup-sized slice of channels
    const size_t total = static_cast<size_t>(L) * N * C;
    for (size_t i = i0; i < total; i += stride) {
        const int c = static_cast<int>(i % C);
        const int n = static_cast<int>((i / C) % N);
        const int j = static_cast<int>(i / (static_cast<size_t>(C) * N));
        int path[L], len = 0;
        for (int v = n; v >= 0 && len < L; v = parent_of(v))
            path[len++] = v;   // leaf first
        const int node = path[len - 1 - (j < len ? j : len - 1)];
        Act xv = static_cast<const Act*>(w.x_nodes)[static_cast<size_t>(node) * C + c];
        if (perturb && n == N - 1 && j == len - 1 && c == 0) {
            if constexpr (sizeof(Act) == 2)
                xv = static_cast<Act>(xv ^ 0x0040u);
            else
                xv = __uint_as_float(__float_as_uint(xv) ^ 0x00400000u);
        }
        static_cast<Act*>(w.x_steps)[i] = xv;
        if (c < Hv) {
            const size_t gi = (static_cast<size_t>(j) * N + n) * Hv + c;
            w.a_steps[gi] = w.a_nodes[static_cast<size_t>(node) * Hv + c];
            w.b_steps[gi] = w.b_nodes[static_cast<size_t>(node) * Hv + c];
        }
    }
}

// Bitwise comparison.  result[1] counts output values that differ, result[2]
// state and tail words that differ (vector atomics on device memory).
template <typename Act>
__global__ __launch_bounds__(256) void compare_kernel(Ws w, int Hv, int D, int C, int32_t* result) {
    const size_t nO = static_cast<size_t>(Hv) * D;
    const size_t nS = static_cast<size_t>(Hv) * D * D;
    const size_t nT = static_cast<size_t>(C) * 4;
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    const size_t i0 = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    int bad_o = 0, bad_s = 0;
    for (size_t i = i0; i < nO * N; i += stride) {
        const int n = static_cast<int>(i / nO);
        int len = 0;
        for (int v = n; v >= 0 && len < L; v = parent_of(v))
            ++len;
        const float t = w.o_tree[i];
        const float d = w.o_steps[static_cast<size_t>(len - 1) * N * nO + i];
        bad_o += __float_as_uint(t) != __float_as_uint(d);
    }
    // sequence CHAIN-1 replays exactly the 8-token committed path
    const float* dec_S = w.states + static_cast<size_t>(CHAIN - 1) * nS;
    for (size_t i = i0; i < nS; i += stride)
        bad_s += __float_as_uint(w.commit_S[i]) != __float_as_uint(dec_S[i]);
    const Act* dec_T = static_cast<const Act*>(L % 2 ? w.tails1 : w.tails0) + static_cast<size_t>(CHAIN - 1) * nT;
    for (size_t i = i0; i < nT; i += stride)
        bad_s += static_cast<const Act*>(w.commit_tail)[i] != dec_T[i];
    if (bad_o)
        atomicAdd(result + 1, bad_o);
    if (bad_s)
        atomicAdd(result + 2, bad_s);
}

__global__ void verdict_kernel(const int32_t* status, int32_t* result) {
    if (threadIdx.x == 0) {
        const bool ok = result[1] == 0 && result[2] == 0 && status[0] == GDN_OK && status[1] == GDN_OK;
        result[3] = status[0] != GDN_OK ? status[0] : status[1];
        result[0] = ok ? GDN_OK : GDN_ERR_SELF_CHECK;
    }
}

template <typename Act>
hipError_t run(const Geo& g0, void* ws, uint32_t seed, int perturb, int32_t* result, hipStream_t s) {
    Ws w;
    carve(g0, ws, &w);
    Geo g1 = g0, gN = g0;
    g1.B = 1;
    gN.B = N;
    const dim3 grid(1024), block(256);
    hipLaunchKernelGGL(gen_kernel<Act>, grid, block, 0, s, w, g0.Hv, g0.D, g0.C, seed, result);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if ((e = launch_tree_verify(g1, w.ckpt, w.ckpt_tail, w.w, N, w.parent, w.x_nodes, w.a_nodes, w.b_nodes, w.o_tree,
                                w.status, w.tree_ws, s)) != hipSuccess)
        return e;
    hipLaunchKernelGGL(expand_kernel<Act>, grid, block, 0, s, w, g0.Hv, g0.D, g0.C, perturb);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    const size_t es = g0.bf16 ? 2 : 4;
    const size_t ob = static_cast<size_t>(N) * g0.Hv * g0.D;
    for (int j = 0; j < L; ++j) {
        void* tin = j % 2 ? w.tails1 : w.tails0;
        void* tout = j % 2 ? w.tails0 : w.tails1;
        const char* xj = static_cast<const char*>(w.x_steps) + static_cast<size_t>(j) * N * g0.C * es;
        if ((e = launch_token(gN, w.states, tin, tout, w.w, xj, w.a_steps + static_cast<size_t>(j) * N * g0.Hv,
                              w.b_steps + static_cast<size_t>(j) * N * g0.Hv, w.o_steps + j * ob, s)) != hipSuccess)
            return e;
    }
    if ((e = launch_commit(g1, w.commit_S, w.commit_tail, w.w, N, w.parent, w.x_nodes, w.a_nodes, w.b_nodes, L, w.path,
                           nullptr, w.status + 1, nullptr, s)) != hipSuccess)
        return e;
    hipLaunchKernelGGL(compare_kernel<Act>, grid, block, 0, s, w, g0.Hv, g0.D, g0.C, result);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL(verdict_kernel, dim3(1), dim3(64), 0, s, w.status, result);
    return hipGetLastError();
}

}  // namespace sc

size_t self_check_ws_bytes(const Geo& g) { return sc::carve(g, reinterpret_cast<void*>(256), nullptr); }

hipError_t launch_self_check(const Geo& g, void* ws, uint32_t seed, int perturb, int32_t* result, hipStream_t s) {
    if (g.bf16)
        return sc::run<uint16_t>(g, ws, seed, perturb, result, s);
    return sc::run<float>(g, ws, seed, perturb, result, s);
}

}  // namespace gdn
