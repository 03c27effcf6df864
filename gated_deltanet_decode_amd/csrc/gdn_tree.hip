// gdn_tree.hip -- tree verify and path commit.
//
// Verify (repository "Architecture" page, decode-loop diagram: one pass over
// the whole draft tree of up to 32 nodes; "Architecture" section 8.1: the
// state must be branched for a tree of guesses) reads the checkpoint state
// once.  Each workgroup owns a block of rows of one value head; a lane keeps
// its slice of the checkpoint row plus a stack of up to 8 branched rows, one
// per tree level, all in registers, and walks the nodes in depth-first
// pre-order so that a node's parent row is always on the stack.  Nothing is
// written but the per-node outputs, so rejecting the round costs nothing.
//
// Commit replays the accepted path from the checkpoint with the same per-token
// arithmetic as decode (gdn_core.hpp), so the committed state is bit-identical
// to token-by-token decode of the path; the tail is rewritten by a second,
// stream-ordered launch after every workgroup of the first has read it.
//
// Per-node conv outputs, normalised q/k and gates are computed once per
// workgroup into LDS: first every thread computes conv outputs for (node,
// channel) pairs, then each wave normalises whole nodes with the same wave
// butterfly as the decode kernel.
#include "gdn_core.hpp"
#include "gdn_launch.hpp"
#include "gdn_tree.hpp"

#include <type_traits>

namespace gdn {

__global__ __launch_bounds__(64) void tree_tables_kernel(int n, const int32_t* __restrict__ parent,
                                                         int32_t* __restrict__ depth, int32_t* __restrict__ order,
                                                         int32_t* __restrict__ status) {
    __shared__ int32_t depth_s[kMaxNodes], order_s[kMaxNodes];
    const bool ok = tree_tables_wave(n, parent, depth_s, order_s);
    __syncthreads();
    const int lane = threadIdx.x;
    if (ok && lane < n) {
        depth[lane] = depth_s[lane];
        order[lane] = order_s[lane];
    }
    if (lane == 0)
        *status = ok ? 0 : 5;
}

hipError_t launch_tree_tables(int n, const int32_t* parent, int32_t* depth, int32_t* order, int32_t* status,
                              hipStream_t s) {
    hipLaunchKernelGGL(tree_tables_kernel, dim3(1), dim3(64), 0, s, n, parent, depth, order, status);
    return hipGetLastError();
}

// Shared-memory image of up to kMaxNodes tokens for one workgroup.
template <int D, int ROWS>
struct NodeSmem {
    float qk[kMaxNodes][2 * D];  // q~|k~ of the workgroup's q/k head, normalised in place
    float v[kMaxNodes][ROWS];    // v of the workgroup's rows
    float kq[kMaxNodes];
    float alpha[kMaxNodes];
    float beta[kMaxNodes];
    int32_t depth[kMaxNodes];
    int32_t order[kMaxNodes];
    int32_t parent[kMaxNodes];
    int32_t ok;
};

// Fill conv outputs, normalised q/k, kq and gates for tokens 0..count-1.
// Token i is node id_of(i) at depth depth_of(i); anc_of(i, k) is its ancestor
// k steps up (only asked for k < depth).
template <int D, int ROWS, typename Act, typename IdOf, typename DepthOf, typename AncOf>
__device__ void fill_nodes(NodeSmem<D, ROWS>& sm, int count, IdOf id_of, DepthOf depth_of, AncOf anc_of,
                           const Act* __restrict__ x, const Act* __restrict__ tail, const Act* __restrict__ w,
                           const float* __restrict__ a, const float* __restrict__ b, int Hk, int Hv, int C, int grp,
                           int h, int row0) {
    constexpr int PER = 2 * D + ROWS;
    for (int idx = threadIdx.x; idx < count * PER; idx += blockDim.x) {
        const int i = idx / PER;
        const int ch = idx % PER;
        const int c = ch < D ? grp * D + ch : ch < 2 * D ? Hk * D + grp * D + (ch - D) : 2 * Hk * D + h * D + row0 + (ch - 2 * D);
        const int node = id_of(i);
        const int d = depth_of(i);
        int anc[3];
#pragma unroll
        for (int k = 1; k <= 3; ++k)
            anc[k - 1] = (k <= d - 1) ? anc_of(i, k) : 0;
        float win[4], wf[4];
        node_window<Act>(x, tail, C, c, node, d, anc, win);
        Quad<Act>::to_float(Quad<Act>::load(w + static_cast<size_t>(c) * 4), wf);
        const float yv = conv_silu(wf, win);
        if (ch < 2 * D)
            sm.qk[i][ch] = yv;
        else
            sm.v[i][ch - 2 * D] = yv;
    }
    __syncthreads();
    constexpr int J = Prep<D>::J;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwaves = blockDim.x / kWave;
    for (int i = wave; i < count; i += nwaves) {
        float qv[J], kv[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int e = lane + kWave * j;
            qv[j] = e < D ? sm.qk[i][e] : 0.0f;
            kv[j] = e < D ? sm.qk[i][D + e] : 0.0f;
        }
        float kq;
        prep_qk<D>(qv, kv, kq);
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int e = lane + kWave * j;
            if (e < D) {
                sm.qk[i][e] = qv[j];
                sm.qk[i][D + e] = kv[j];
            }
        }
        if (lane == 0) {
            const int node = id_of(i);
            float al, be;
            gates(a[static_cast<size_t>(node) * Hv + h], b[static_cast<size_t>(node) * Hv + h], al, be);
            sm.kq[i] = kq;
            sm.alpha[i] = al;
            sm.beta[i] = be;
        }
    }
    __syncthreads();
}

// ------------------------------------------------------------ verify

template <int D, typename Act>
__global__ __launch_bounds__(256) void tree_verify_kernel(const float* __restrict__ Sc, const Act* __restrict__ tail,
                                                          const Act* __restrict__ w, int n,
                                                          const int32_t* __restrict__ parent,
                                                          const Act* __restrict__ x, const float* __restrict__ a,
                                                          const float* __restrict__ b, float* __restrict__ o,
                                                          int32_t* __restrict__ status, int Hk, int Hv, int C,
                                                          int blocks_per_head) {
    using R = Row<D>;
    constexpr int NV = R::NV, LPR = R::LPR, RPW = R::RPW;
    constexpr int ROWS = 4 * RPW;
    __shared__ NodeSmem<D, ROWS> sm;

    const int blk = blockIdx.x % blocks_per_head;
    const int h = blockIdx.x / blocks_per_head;
    const int grp = h / (Hv / Hk);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r = lane % LPR;
    const int row0 = blk * ROWS;
    const int lrow = wave * RPW + lane / LPR;
    const int row = row0 + lrow;

    const float* Sh = Sc + static_cast<size_t>(h) * D * D;
    float4 base[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j)
        base[j] = *reinterpret_cast<const float4*>(Sh + row * D + R::key(j, r));

    if (wave == 0) {
        const bool ok = tree_tables_wave(n, parent, sm.depth, sm.order);
        if (lane < n)
            sm.parent[lane] = ok ? parent[lane] : -1;
        if (lane == 0) {
            sm.ok = ok ? 1 : 0;
            if (status && blockIdx.x == 0)
                *status = ok ? 0 : 5;
        }
    }
    __syncthreads();
    if (!sm.ok)
        return;

    const int32_t* par = sm.parent;
    fill_nodes<D, ROWS, Act>(
        sm, n, [](int i) { return i; }, [&](int i) { return sm.depth[i]; },
        [&](int i, int k) {
            int m = i;
            for (int s = 0; s < k; ++s)
                m = par[m];
            return m;
        },
        x, tail, w, a, b, Hk, Hv, C, grp, h, row0);

    float4 stack[kMaxDepth][NV];
#pragma unroll
    for (int l = 0; l < kMaxDepth; ++l)
#pragma unroll
        for (int j = 0; j < NV; ++j)
            stack[l][j] = base[j];

    float4 kk[NV], qq[NV], cur[NV];
    for (int it = 0; it < n; ++it) {
        const int node = sm.order[it];
        const int d = sm.depth[node];
#pragma unroll
        for (int j = 0; j < NV; ++j)
            cur[j] = base[j];
#pragma unroll
        for (int l = 0; l < kMaxDepth - 1; ++l)
            if (l == d - 2)
#pragma unroll
                for (int j = 0; j < NV; ++j)
                    cur[j] = stack[l][j];
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            kk[j] = *reinterpret_cast<const float4*>(&sm.qk[node][D + R::key(j, r)]);
            qq[j] = *reinterpret_cast<const float4*>(&sm.qk[node][R::key(j, r)]);
        }
        const float out = row_update<D>(cur, kk, qq, sm.alpha[node], sm.beta[node], sm.v[node][lrow], sm.kq[node]);
#pragma unroll
        for (int l = 0; l < kMaxDepth; ++l)
            if (l == d - 1)
#pragma unroll
                for (int j = 0; j < NV; ++j)
                    stack[l][j] = cur[j];
        if (r == 0)
            o[(static_cast<size_t>(node) * Hv + h) * D + row] = out;
    }
}

// Runs f(D, Act) for the geometry's head width and activation type.
template <typename F>
static hipError_t dispatch(const Geo& g, F&& f) {
    if (g.D == 128) {
        if (g.bf16)
            f(std::integral_constant<int, 128>{}, uint16_t{});
        else
            f(std::integral_constant<int, 128>{}, float{});
    } else {
        if (g.bf16)
            f(std::integral_constant<int, 32>{}, uint16_t{});
        else
            f(std::integral_constant<int, 32>{}, float{});
    }
    return hipGetLastError();
}

hipError_t launch_tree_verify(const Geo& g, const float* S, const void* tail, const void* w, int n,
                              const int32_t* parent, const void* x, const float* a, const float* b, float* o,
                              int32_t* status, hipStream_t s) {
    return dispatch(g, [&](auto dtag, auto atag) {
        constexpr int D = decltype(dtag)::value;
        using Act = decltype(atag);
        const int bph = D / (4 * Row<D>::RPW);
        hipLaunchKernelGGL((tree_verify_kernel<D, Act>), dim3(static_cast<unsigned>(g.Hv * bph)), dim3(256), 0, s,
                           S, static_cast<const Act*>(tail), static_cast<const Act*>(w), n, parent,
                           static_cast<const Act*>(x), a, b, o, status, g.Hk, g.Hv, g.C, bph);
    });
}

// ------------------------------------------------------------ commit

template <int D, typename Act>
__global__ __launch_bounds__(256) void commit_state_kernel(float* __restrict__ S, const Act* __restrict__ tail,
                                                           const Act* __restrict__ w, int n,
                                                           const int32_t* __restrict__ parent,
                                                           const Act* __restrict__ x, const float* __restrict__ a,
                                                           const float* __restrict__ b, int L,
                                                           const int32_t* __restrict__ path, float* __restrict__ o,
                                                           int32_t* __restrict__ status, int Hk, int Hv, int C,
                                                           int blocks_per_head) {
    using R = Row<D>;
    constexpr int NV = R::NV, LPR = R::LPR, RPW = R::RPW;
    constexpr int ROWS = 4 * RPW;
    __shared__ NodeSmem<D, ROWS> sm;

    const int blk = blockIdx.x % blocks_per_head;
    const int h = blockIdx.x / blocks_per_head;
    const int grp = h / (Hv / Hk);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r = lane % LPR;
    const int row0 = blk * ROWS;
    const int lrow = wave * RPW + lane / LPR;
    const int row = row0 + lrow;

    float* Sh = S + static_cast<size_t>(h) * D * D;
    float4 cur[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j)
        cur[j] = *reinterpret_cast<const float4*>(Sh + row * D + R::key(j, r));

    if (wave == 0) {
        bool ok = tree_tables_wave(n, parent, nullptr, nullptr);
        ok = ok && path_check_wave(n, parent, L, path);
        if (lane < L)
            sm.order[lane] = ok ? path[lane] : 0;
        if (lane == 0) {
            sm.ok = ok ? 1 : 0;
            if (status && blockIdx.x == 0)
                *status = ok ? 0 : 5;
        }
    }
    __syncthreads();
    if (!sm.ok)
        return;

    fill_nodes<D, ROWS, Act>(
        sm, L, [&](int i) { return sm.order[i]; }, [](int i) { return i + 1; },
        [&](int i, int k) { return sm.order[i - k]; }, x, tail, w, a, b, Hk, Hv, C, grp, h, row0);

    float4 kk[NV], qq[NV];
    for (int i = 0; i < L; ++i) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            kk[j] = *reinterpret_cast<const float4*>(&sm.qk[i][D + R::key(j, r)]);
            qq[j] = *reinterpret_cast<const float4*>(&sm.qk[i][R::key(j, r)]);
        }
        const float out = row_update<D>(cur, kk, qq, sm.alpha[i], sm.beta[i], sm.v[i][lrow], sm.kq[i]);
        if (o && r == 0)
            o[(static_cast<size_t>(i) * Hv + h) * D + row] = out;
    }
#pragma unroll
    for (int j = 0; j < NV; ++j)
        *reinterpret_cast<float4*>(Sh + row * D + R::key(j, r)) = cur[j];
}

// The tail after a commit holds the last four raw inputs of (old tail ++ path).
template <typename Act>
__global__ __launch_bounds__(256) void commit_tail_kernel(Act* __restrict__ tail, int n,
                                                          const int32_t* __restrict__ parent,
                                                          const Act* __restrict__ x, int L,
                                                          const int32_t* __restrict__ path, int C) {
    __shared__ int32_t ok_s;
    __shared__ int32_t path_s[kMaxDepth];
    if (threadIdx.x < kWave) {
        bool ok = tree_tables_wave(n, parent, nullptr, nullptr);
        ok = ok && path_check_wave(n, parent, L, path);
        if (threadIdx.x < L)
            path_s[threadIdx.x] = ok ? path[threadIdx.x] : 0;
        if (threadIdx.x == 0)
            ok_s = ok ? 1 : 0;
    }
    __syncthreads();
    const int c = blockIdx.x * blockDim.x + threadIdx.x;
    if (!ok_s || c >= C)
        return;
    using Q = Quad<Act>;
    typename Q::raw t = Q::load(tail + static_cast<size_t>(c) * 4);
    for (int j = 0; j < L; ++j)
        t = Q::push(t, x[static_cast<size_t>(path_s[j]) * C + c]);
    Q::store(tail + static_cast<size_t>(c) * 4, t);
}

hipError_t launch_commit(const Geo& g, float* S, void* tail, const void* w, int n, const int32_t* parent,
                         const void* x, const float* a, const float* b, int L, const int32_t* path, float* o,
                         int32_t* status, hipStream_t s) {
    hipError_t e = dispatch(g, [&](auto dtag, auto atag) {
        constexpr int D = decltype(dtag)::value;
        using Act = decltype(atag);
        const int bph = D / (4 * Row<D>::RPW);
        hipLaunchKernelGGL((commit_state_kernel<D, Act>), dim3(static_cast<unsigned>(g.Hv * bph)), dim3(256), 0,
                           s, S, static_cast<const Act*>(tail), static_cast<const Act*>(w), n, parent,
                           static_cast<const Act*>(x), a, b, L, path, o, status, g.Hk, g.Hv, g.C, bph);
    });
    if (e != hipSuccess)
        return e;
    const dim3 grid(static_cast<unsigned>((g.C + 255) / 256)), block(256);
    if (g.bf16)
        hipLaunchKernelGGL(commit_tail_kernel<uint16_t>, grid, block, 0, s, static_cast<uint16_t*>(tail), n, parent,
                           static_cast<const uint16_t*>(x), L, path, g.C);
    else
        hipLaunchKernelGGL(commit_tail_kernel<float>, grid, block, 0, s, static_cast<float*>(tail), n, parent,
                           static_cast<const float*>(x), L, path, g.C);
    return hipGetLastError();
}

}  // namespace gdn
