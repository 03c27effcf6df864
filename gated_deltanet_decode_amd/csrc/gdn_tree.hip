// gdn_tree.hip -- tree verify, path commit, and block verify / commit.
//
// Verify (repository "Architecture" page, decode-loop diagram: one pass over
// the whole draft tree of up to 32 nodes; "Architecture" section 8.1: the
// state must be branched for a tree of guesses) reads each sequence's
// checkpoint state once and writes nothing but the per-node outputs, so
// rejecting the round costs nothing.  A batch holds one tree per sequence.
// Two launches:
//   tree_prep_kernel    one workgroup per sequence builds its tree tables
//                       (validity, pre-order, depths); the others, one per
//                       (sequence, q/k head, 1 or 4 nodes), compute the conv
//                       window over each node's ancestors and the tail, the
//                       q/k norm and the gates, into a caller-owned workspace;
//   tree_verify_kernel  each workgroup owns a block of rows of one value head
//                       and walks its tree in depth-first pre-order.  A
//                       lane's slice of the current row stays in registers;
//                       the row after each node is saved in an LDS slot per
//                       tree level, from which a later sibling's subtree
//                       restarts.  Node operands stream from the workspace
//                       through a register ring several nodes ahead.
// A block (the "Architecture" page's parts list: delta-rule kernels for one
// token, a block and a tree) is the chain 0 -> 1 -> ... -> k-1: the same two
// launches with no parent array, no tables to check and no saved levels.
// Committing a block prefix streams each state once, replaying the prefix's
// prepared operands from LDS, and rewrites the conv tail in the same launch.
//
// Commit of a tree path replays the accepted path from the checkpoint with
// the same per-token arithmetic as decode (gdn_core.hpp), so the committed
// state is bit-identical to token-by-token decode of the path.  Its per-token
// operands are computed per workgroup into LDS, or read from the verify's
// workspace; in the first form the tail is rewritten by a second,
// stream-ordered launch after every workgroup of the first has read it.
#include "gdn_core.hpp"
#include "gdn_launch.hpp"
#include "gdn_tree.hpp"

#include <type_traits>
#include <utility>

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

// Shared-memory image of up to MAXN tokens (tree nodes or path positions) for
// one workgroup: the workgroup's channels are its q/k head's q and k channels
// and the v channels of its rows.
template <int D, int ROWS, int MAXN, typename Act>
struct alignas(16) NodeSmem {
    static constexpr int PER = 2 * D + ROWS;
    float qk[MAXN][2 * D];      // q~|k~ of each token, normalised in place
    float v[MAXN][ROWS];        // v of the workgroup's rows
    float wl[PER][4];           // conv weights of the workgroup's channels
    float kq[MAXN], alpha[MAXN], beta[MAXN];
    float ga[MAXN], gb[MAXN];   // raw gate inputs of the value head
    Act xr[MAXN][PER];          // raw inputs of the workgroup's channels
    Act tl[PER][4];             // checkpoint conv tail of those channels
    int32_t node[MAXN];         // node id of token i
    int32_t depth[MAXN];        // depth of token i (root = 1)
    int32_t anc[MAXN][3];       // token index of the ancestor 1..3 steps up, -1 past the root
    int32_t order[MAXN];        // depth-first pre-order of the tokens (verify)
    int32_t ok;
    int32_t len;                // tokens of the accepted path (commit)
};

// Conv outputs, normalised q/k, k.q and gates for tokens 0..count-1 (from
// sm.node, sm.depth and sm.anc), in two steps so that the caller can overlap
// other work with the loads: fill_issue requests every global input into
// registers at once (each thread its channels' raw inputs at every token),
// fill_finish stores them to LDS, convolves, normalises and computes gates.
template <int D, int ROWS, int MAXN, typename Act>
struct FillRegs {
    static constexpr int PER = NodeSmem<D, ROWS, MAXN, Act>::PER;
    static constexpr int SLOTS = (PER + 255) / 256;
    Act r[SLOTS][MAXN];
    typename Quad<Act>::raw tq[SLOTS], wq[SLOTS];
    float ga, gb;
};

template <int D, int ROWS, int MAXN, typename Act>
__device__ __forceinline__ void fill_issue(FillRegs<D, ROWS, MAXN, Act>& f, const NodeSmem<D, ROWS, MAXN, Act>& sm,
                                           int count, const Act* __restrict__ x, const Act* __restrict__ tail,
                                           const Act* __restrict__ w, const float* __restrict__ a,
                                           const float* __restrict__ b, int Hk, int Hv, int C, int grp, int h,
                                           int row0) {
    constexpr int PER = FillRegs<D, ROWS, MAXN, Act>::PER;
    {
        const int i = threadIdx.x < count ? threadIdx.x : count - 1;
        const size_t gi = static_cast<size_t>(sm.node[i < MAXN ? i : MAXN - 1]) * Hv + h;
        f.ga = a[gi];
        f.gb = b[gi];
    }
#pragma unroll
    for (int k = 0; k < FillRegs<D, ROWS, MAXN, Act>::SLOTS; ++k) {
        const int ch0 = threadIdx.x + 256 * k;
        const int ch = ch0 < PER ? ch0 : PER - 1;   // clamped: loads stay unconditional
        const int c = ch < D ? grp * D + ch : ch < 2 * D ? Hk * D + grp * D + (ch - D) : 2 * Hk * D + h * D + row0 + (ch - 2 * D);
#pragma unroll
        for (int i = 0; i < MAXN; ++i)
            f.r[k][i] = x[static_cast<size_t>(sm.node[i < count ? i : count - 1]) * C + c];
        f.tq[k] = Quad<Act>::load(tail + static_cast<size_t>(c) * 4);
        f.wq[k] = Quad<Act>::load(w + static_cast<size_t>(c) * 4);
    }
}

template <int D, int ROWS, int MAXN, typename Act>
__device__ void fill_finish(const FillRegs<D, ROWS, MAXN, Act>& f, NodeSmem<D, ROWS, MAXN, Act>& sm, int count) {
    constexpr int PER = FillRegs<D, ROWS, MAXN, Act>::PER;
    if (threadIdx.x < MAXN) {
        sm.ga[threadIdx.x] = f.ga;
        sm.gb[threadIdx.x] = f.gb;
    }
#pragma unroll
    for (int k = 0; k < FillRegs<D, ROWS, MAXN, Act>::SLOTS; ++k) {
        const int ch = threadIdx.x + 256 * k;
        if (ch < PER) {
            float wf[4];
            Quad<Act>::to_float(f.wq[k], wf);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sm.tl[ch][j] = Quad<Act>::elem(f.tq[k], j);
                sm.wl[ch][j] = wf[j];
            }
#pragma unroll
            for (int i = 0; i < MAXN; ++i)
                if (i < count)
                    sm.xr[i][ch] = f.r[k][i];
        }
    }
    __syncthreads();
    // conv + SiLU per (token, channel), from LDS only
    for (int idx = threadIdx.x; idx < count * PER; idx += blockDim.x) {
        const int i = idx / PER;
        const int ch = idx % PER;
        const int d = sm.depth[i];
        float win[4];
        win[3] = widen(sm.xr[i][ch]);
#pragma unroll
        for (int k = 1; k <= 3; ++k) {
            const int an = sm.anc[i][k - 1];
            const Act* src = an >= 0 ? &sm.xr[an][ch] : &sm.tl[ch][3 + d - k];
            win[3 - k] = widen(*src);
        }
        const float yv = conv_silu(sm.wl[ch], win);
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
            float al, be;
            gates(sm.ga[i], sm.gb[i], al, be);
            sm.kq[i] = kq;
            sm.alpha[i] = al;
            sm.beta[i] = be;
        }
    }
    __syncthreads();
}

// One token's operands for a lane's row slice.
template <int D>
struct TokOps {
    float4 k[Row<D>::NV], q[Row<D>::NV];
    float v, alpha, beta, kq;
};

template <int D, int ROWS, int MAXN, typename Act>
__device__ __forceinline__ void tok_load(TokOps<D>& t, const NodeSmem<D, ROWS, MAXN, Act>& sm, int i, int r,
                                         int lrow) {
#pragma unroll
    for (int j = 0; j < Row<D>::NV; ++j) {
        t.k[j] = *reinterpret_cast<const float4*>(&sm.qk[i][D + Row<D>::key(j, r)]);
        t.q[j] = *reinterpret_cast<const float4*>(&sm.qk[i][Row<D>::key(j, r)]);
    }
    t.v = sm.v[i][lrow];
    t.alpha = sm.alpha[i];
    t.beta = sm.beta[i];
    t.kq = sm.kq[i];
}

// ------------------------------------------------------------ verify

// Per-node operands of the batch's trees, prepared once by tree_prep_kernel
// (node index m = sequence * n + node):
//   qk   f32 [B*n][Hk][2*D]  q^ | k^ of each q/k head (normalised)
//   v    f32 [B*n][Hv][D]    conv output of each value head's v channels
//   abk  f32 [B*n][Hv][4]    alpha, beta, k^.q^ of the value head's q/k head, 0
//   tab  i32 [B][2n+1]       per sequence: the node at each pre-order position,
//                            the depth at each position, then 1 if the tree is
//                            valid (0 otherwise)
// abk holds (alpha, beta, k^.q^, 0) per (node, value head): the walk loads
// it with a lane-dependent address, so it is a vector load counted with the
// other vector loads rather than a scalar load sharing the LDS counter.
struct TreeWs {
    float *qk, *v, *abk;
    int32_t* tab;
};

size_t tree_ws_bytes(int B, int n, int Hk, int Hv, int D) {
    const size_t m = static_cast<size_t>(B) * n;
    return m * (2ull * Hk * D + static_cast<size_t>(Hv) * D + 4ull * Hv) * 4 +
           static_cast<size_t>(B) * (2 * n + 1) * 4 + 4 * 256;
}

static TreeWs tree_ws_carve(void* base, int B, int n, int Hk, int Hv, int D) {
    auto align = [](uintptr_t p) { return (p + 255) & ~static_cast<uintptr_t>(255); };
    uintptr_t p = align(reinterpret_cast<uintptr_t>(base));
    const size_t m = static_cast<size_t>(B) * n;
    TreeWs w;
    auto take = [&](size_t cnt) { void* r = reinterpret_cast<void*>(p); p = align(p + cnt * 4); return r; };
    w.qk = static_cast<float*>(take(m * Hk * 2 * D));
    w.v = static_cast<float*>(take(m * Hv * D));
    w.abk = static_cast<float*>(take(m * Hv * 4));
    w.tab = static_cast<int32_t*>(take(static_cast<size_t>(B) * (2 * n + 1)));
    return w;
}

// Workgroups 0 .. B-1 build each sequence's tree tables (validity, pre-order,
// depths) once for every workgroup of the verify kernel, and report the
// sequence's status.  The others, one per (sequence, q/k head, node): the
// node's conv window over its q/k head's channels and its value heads'
// channels, the q/k norm and the gates.  With no parent array the nodes are a
// block, the chain 0 -> 1 -> ... -> n-1 (valid by construction).  Each
// workgroup prepares NPW consecutive nodes of one (sequence, q/k head), all
// their window loads in flight together: NPW = 1 when the grid is small (one
// tree), 4 when it is many workgroups deep, where one node per workgroup would
// leave each CU waiting through several latency-bound rounds.
// The ancestor chain is followed at most three links and every link is
// checked, so a malformed parent array stays in bounds (the verify kernel
// reports it and writes nothing).
template <int D, typename Act, int NPW>
__device__ __forceinline__ void tree_prep_body(int bid, const Act* __restrict__ tail, const Act* __restrict__ w,
                                               int n, const int32_t* __restrict__ parent,
                                               const Act* __restrict__ x, const float* __restrict__ a,
                                               const float* __restrict__ b, TreeWs ws,
                                               int32_t* __restrict__ status, int B, int Hk, int Hv, int C) {
    static_assert(NPW >= 1 && NPW <= 4, "one wave normalises each node of the workgroup");
    // The index arithmetic is made to depend on every argument, so all the
    // argument loads issue together (one kernel-argument round trip).
    asm volatile("" : "+s"(B) : "s"(tail), "s"(w), "s"(n), "s"(parent), "s"(x), "s"(a), "s"(b), "s"(ws.qk),
                 "s"(ws.v), "s"(ws.abk), "s"(ws.tab), "s"(status), "s"(Hk), "s"(Hv), "s"(C));
    __shared__ float yqk[NPW][2 * D];
    __shared__ int32_t anc_s[NPW][4];
    __shared__ int32_t depth_s[kMaxNodes], order_s[kMaxNodes];
    if (bid < B) {
        const int bq = bid;
        if (parent == nullptr) {
            int32_t* tab = ws.tab + static_cast<size_t>(bq) * (2 * n + 1);
            const int t = threadIdx.x;
            if (t < n) {
                tab[t] = t;
                tab[n + t] = t + 1;
            }
            if (t == 0)
                tab[2 * n] = 1;
            return;
        }
        bool ok = false;
        if (threadIdx.x < kWave)
            ok = tree_tables_wave(n, parent + static_cast<size_t>(bq) * n, depth_s, order_s);
        __syncthreads();
        if (threadIdx.x < kWave) {
            const int lane = threadIdx.x;
            int32_t* tab = ws.tab + static_cast<size_t>(bq) * (2 * n + 1);
            if (ok && lane < n) {
                const int node = order_s[lane];
                tab[lane] = node;
                tab[n + lane] = depth_s[node];
            }
            if (lane == 0) {
                tab[2 * n] = ok ? 1 : 0;
                if (status)
                    status[bq] = ok ? 0 : 5;
            }
        }
        return;
    }
    const int wg = bid - B;
    const int nq = (n + NPW - 1) / NPW;   // node groups per (sequence, q/k head)
    const int i0 = (wg % nq) * NPW;       // the workgroup's first node
    const int g = (wg / nq) % Hk;
    const int bq = wg / (nq * Hk);
    const int G = Hv / Hk;
    const int m0 = bq * n;   // workspace index of the sequence's node 0
    x += static_cast<size_t>(m0) * C;
    a += static_cast<size_t>(m0) * Hv;
    b += static_cast<size_t>(m0) * Hv;
    tail += static_cast<size_t>(bq) * C * 4;
    const int lane = threadIdx.x & (kWave - 1);
    if (threadIdx.x < kWave && parent != nullptr) {
        const int p = lane < n ? parent[m0 + lane] : -1;
#pragma unroll
        for (int u = 0; u < NPW; ++u) {
            int cur = i0 + u < n ? i0 + u : n - 1, m = 0;
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const int up = __shfl(p, cur >= 0 ? cur : 0, kWave);
                const bool link = cur >= 0 && up >= 0 && up < cur;
                if (lane == 0)
                    anc_s[u][k] = link ? up : -1;
                m += link ? 1 : 0;
                cur = link ? up : -1;
            }
            if (lane == 0)
                anc_s[u][3] = m;   // ancestors found (at most 3)
        }
    } else if (parent == nullptr && threadIdx.x < NPW) {   // a block: the previous positions
        const int u = threadIdx.x;
        const int i = i0 + u < n ? i0 + u : n - 1;
#pragma unroll
        for (int k = 0; k < 3; ++k)
            anc_s[u][k] = i - 1 - k >= 0 ? i - 1 - k : -1;
        anc_s[u][3] = i < 3 ? i : 3;
    }
    __syncthreads();
    // Every window load of the workgroup's nodes is issued before the first is used.
    for (int ch = threadIdx.x; ch < (2 + G) * D; ch += blockDim.x) {
        const int c = ch < D ? g * D + ch : ch < 2 * D ? Hk * D + g * D + (ch - D) : 2 * Hk * D + G * g * D + (ch - 2 * D);
        float win[NPW][4], wf[4];
#pragma unroll
        for (int u = 0; u < NPW; ++u) {
            const int i = i0 + u < n ? i0 + u : n - 1;
            const int m = anc_s[u][3];
            win[u][3] = widen(x[static_cast<size_t>(i) * C + c]);
#pragma unroll
            for (int k = 1; k <= 3; ++k) {
                const Act* src = (k <= m) ? x + static_cast<size_t>(anc_s[u][k - 1]) * C + c
                                          : tail + static_cast<size_t>(c) * 4 + (4 + m - k);
                win[u][3 - k] = widen(*src);
            }
        }
        Quad<Act>::to_float(Quad<Act>::load(w + static_cast<size_t>(c) * 4), wf);
#pragma unroll
        for (int u = 0; u < NPW; ++u) {
            const int i = i0 + u;
            if (i >= n)
                break;
            const float yv = conv_silu(wf, win[u]);
            if (ch < 2 * D)
                yqk[u][ch] = yv;
            else
                ws.v[(static_cast<size_t>(m0 + i) * Hv + G * g) * D + (ch - 2 * D)] = yv;
        }
    }
    if (threadIdx.x < NPW * G) {
        const int u = threadIdx.x / G, i = i0 + u;
        const int h = G * g + threadIdx.x % G;
        if (i < n) {
            float al, be;
            gates(a[static_cast<size_t>(i) * Hv + h], b[static_cast<size_t>(i) * Hv + h], al, be);
            ws.abk[(static_cast<size_t>(m0 + i) * Hv + h) * 4] = al;
            ws.abk[(static_cast<size_t>(m0 + i) * Hv + h) * 4 + 1] = be;
            ws.abk[(static_cast<size_t>(m0 + i) * Hv + h) * 4 + 3] = 0.0f;
        }
    }
    __syncthreads();
    // Wave u normalises node i0 + u.
    const int u = threadIdx.x / kWave, i = i0 + u;
    if (u < NPW && i < n) {
        constexpr int J = Prep<D>::J;
        float qv[J], kv[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int e = lane + kWave * j;
            qv[j] = e < D ? yqk[u][e] : 0.0f;
            kv[j] = e < D ? yqk[u][D + e] : 0.0f;
        }
        float kq;
        prep_qk<D>(qv, kv, kq);
        float* dst = ws.qk + (static_cast<size_t>(m0 + i) * Hk + g) * 2 * D;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int e = lane + kWave * j;
            if (e < D) {
                dst[e] = qv[j];
                dst[D + e] = kv[j];
            }
        }
        if (lane < G)
            ws.abk[(static_cast<size_t>(m0 + i) * Hv + G * g + lane) * 4 + 2] = kq;
    }
}

// Workgroup bid < B builds sequence bid's tables; the rest prepare node operands.
template <int D, typename Act, int NPW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8))) void tree_prep_kernel(const Act* __restrict__ tail, const Act* __restrict__ w,
                                                        int n, const int32_t* __restrict__ parent,
                                                        const Act* __restrict__ x, const float* __restrict__ a,
                                                        const float* __restrict__ b, TreeWs ws,
                                                        int32_t* __restrict__ status, int B, int Hk, int Hv, int C) {
    tree_prep_body<D, Act, NPW>(blockIdx.x, tail, w, n, parent, x, a, b, ws, status, B, Hk, Hv, C);
}


// The branched rows are kept per tree level below the deepest: the slot of
// depth L holds, for every lane, its slice of the row after the most recent
// node of depth L on the walk.  A node whose parent is the previous node of
// the walk takes the rows still in registers; any other node reloads its
// parent's slot.
template <int D, int LEVELS>
struct alignas(16) VerifySmem {
    float4 stack[LEVELS][Row<D>::NV][256];
};

template <int D>
struct NodeOps {
    float4 k[Row<D>::NV], q[Row<D>::NV];
    float v, abk;   // abk: lane l holds element l % 4 of (alpha, beta, k^.q^, 0)
};

// Value of lane 4 (l / 4) + E in lane l: broadcasts one element of abk.  Every
// lane is written, so the move needs no initial value.
template <int E>
__device__ __forceinline__ float quad_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), E * 0x55, 0xF, 0xF, true));
}

// What a verify workgroup knows about itself: its rows, its sequence's tables
// (built by the prep launch; lane l holds the node at pre-order position l and
// its depth), and where its node operands and outputs are.
template <int D>
struct VerifyCtx {
    using R = Row<D>;
    static constexpr int NV = R::NV, LPR = R::LPR, RPW = R::RPW, ROWS = 4 * RPW;
    int h, grp, bq, lane, r, row, m0, n, Hk, Hv, ord_l, dep_l, ok;
    const float* Sh;
    float* oh;   // o of this lane's row at node 0 of the sequence
    TreeWs ws;

    __device__ VerifyCtx(const float* Sc, int n_, TreeWs ws_, float* o, int Hk_, int Hv_, int blocks_per_head)
        : n(n_), Hk(Hk_), Hv(Hv_), ws(ws_) {
        // Workgroups of one (sequence, q/k head) share their node operands;
        // they are kept on one XCD.
        const int wid = xcd_packed_id(blockIdx.x, gridDim.x);
        const int blk = wid % blocks_per_head;
        h = (wid / blocks_per_head) % Hv;
        bq = wid / (blocks_per_head * Hv);
        grp = h / (Hv / Hk);
        lane = threadIdx.x & (kWave - 1);
        r = lane % LPR;
        row = blk * ROWS + static_cast<int>(threadIdx.x / kWave) * RPW + lane / LPR;
        m0 = bq * n;
        Sh = Sc + (static_cast<size_t>(bq) * Hv + h) * D * D;
        oh = o + (static_cast<size_t>(m0) * Hv + h) * D + row;
        const int32_t* tab = ws.tab + static_cast<size_t>(bq) * (2 * n + 1);
        ok = tab[2 * n];
        ord_l = lane < n ? tab[lane] : 0;
        ord_l = ord_l < 0 ? 0 : ord_l >= n ? n - 1 : ord_l;
        dep_l = lane < n ? tab[n + lane] : 1;
    }
    // Operands of the node at pre-order position `it` (clamped into the tree).
    __device__ __forceinline__ void load_node(NodeOps<D>& t, int it) const {
        const int i = m0 + __builtin_amdgcn_readlane(ord_l, it < n ? it : n - 1);
        const float* qk = ws.qk + (static_cast<size_t>(i) * Hk + grp) * 2 * D;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            t.k[j] = *reinterpret_cast<const float4*>(qk + D + R::key(j, r));
            t.q[j] = *reinterpret_cast<const float4*>(qk + R::key(j, r));
        }
        t.v = ws.v[(static_cast<size_t>(i) * Hv + h) * D + row];
        t.abk = ws.abk[(static_cast<size_t>(i) * Hv + h) * 4 + (lane & 3)];
    }
    // Every lane of a row holds the same sum (the butterfly adds commuted
    // pairs), so all of them store it: no exec branch.
    __device__ __forceinline__ void store_o(int it, float v) const {
        oh[static_cast<size_t>(__builtin_amdgcn_readlane(ord_l, it)) * Hv * D] = v;
    }
};

template <int D>
__device__ __forceinline__ float node_update(float4 (&s)[Row<D>::NV], const NodeOps<D>& t) {
    return row_update<D>(s, t.k, t.q, quad_bcast<0>(t.abk), quad_bcast<1>(t.abk), t.v, quad_bcast<2>(t.abk));
}

// Calls f(integral_constant<I>) for I = 0, 1, ... until one returns false.
template <typename F, int... I>
__device__ __forceinline__ void walk_all(F& f, std::integer_sequence<int, I...>) {
    (void)(f(std::integral_constant<int, I>{}) && ...);
}

// Two forms of the walk.  Both store each node's output as soon as it is
// computed, so the stores overlap the rest of the walk.
//
// Alone on its CU (a batch of one tree) a workgroup needs a deep operand ring
// to hide the fetch latency, and has the LDS for every saved level.
//
// With several trees per CU, occupancy hides the latency, and the walk is
// bound by issue of the VALU and of the operand loads: four waves per SIMD
// (at most 128 VGPRs and 40 KB of LDS per workgroup) and a 3-slot ring.
// Saved levels are kept for depths 1 .. 5 only; a node whose parent is deeper
// and is not the previous node replays its ancestors below depth 5 from the
// depth-5 row, with the same operands and arithmetic, so its row is the same
// bits.  (In random 32-node trees of depth 8 about one node in sixty does.)
struct WalkDeep {
    static constexpr int ring = 6, levels = kMaxDepth - 1, waves = 1;
};
struct WalkWide {
    static constexpr int ring = 3, levels = kMaxDepth - 3, waves = 4;
};

// What a walk does.  Tree: verify a draft tree (saved levels, reloads).
// Chain: verify a block, the chain 0 -> 1 -> ... -> n-1 (every node continues
// from the previous one: no saved levels, no LDS).
enum class WalkKind { Tree, Chain };

struct NoSmem {};

template <int D, typename Walk, WalkKind KIND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(Walk::waves))) void tree_verify_kernel(
    const float* __restrict__ Sc, int n, TreeWs ws, float* __restrict__ o, int Hk, int Hv, int blocks_per_head) {
    using R = Row<D>;
    constexpr int NV = R::NV, RING = Walk::ring, LEVELS = Walk::levels;
    constexpr bool TREE = KIND == WalkKind::Tree;
    using Smem = std::conditional_t<TREE, VerifySmem<D, LEVELS>, NoSmem>;
    __shared__ Smem sm;
    // The index arithmetic is made to depend on every argument, so all the
    // argument loads issue together (one kernel-argument round trip).
    asm volatile("" : "+s"(blocks_per_head) : "s"(Sc), "s"(n), "s"(ws.qk), "s"(ws.v), "s"(ws.abk), "s"(ws.tab), "s"(o),
                 "s"(Hk), "s"(Hv));
    const VerifyCtx<D> c(Sc, n, ws, o, Hk, Hv, blocks_per_head);
    const int tid = threadIdx.x;
    float4 base[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j)
        base[j] = load_stream(c.Sh + c.row * D + R::key(j, c.r));
    if (!c.ok)   // nothing is written for a malformed tree
        return;
    const int len = n;   // walk steps

    // Node operands stream through a ring of RING register slots, unrolled so
    // that each slot keeps its registers: a slot is refilled with the node
    // RING steps ahead as soon as its node is done, which hides the cross-XCD
    // fetch.
    NodeOps<D> ring[RING];
#pragma unroll
    for (int p = 0; p < RING; ++p)
        c.load_node(ring[p], p);
    float4 s[NV];
    // This thread's slot of the level saved after a node of depth e is at
    // base + (e - 1) * kLevelBytes (+ j * 4 KB for vector j).  Bases biased by
    // the depth offsets make each access one add of the uniform d * kLevelBytes
    // (the vector index fits the instruction's unsigned offset).
    constexpr int kLevelBytes = NV * 256 * 16;
    char* save_base = nullptr;     // slot of depth d is save_base + d * kLevelBytes
    char* parent_base = nullptr;   // slot of depth d - 1 is parent_base + d * kLevelBytes
    if constexpr (TREE) {
        char* base = reinterpret_cast<char*>(&sm.stack[0][0][tid]);
        save_base = base - kLevelBytes;
        parent_base = base - 2 * kLevelBytes;
    }
    int dprev = 0;
    // One walk step per node, expanded at compile time (at most kMaxNodes),
    // so that ring slots are static registers and every wait on a slot counts
    // exactly the loads issued after it.
    auto step = [&](auto itc) -> bool {
        constexpr int it = decltype(itc)::value;
        constexpr int p = it % RING;
        if (it >= len)
            return false;
        const int d = __builtin_amdgcn_readlane(c.dep_l, it);
        // A valid tree's pre-order starts at the root, the only node of depth
        // 1, so only the first step starts from the checkpoint rows.
        if constexpr (it == 0) {
#pragma unroll
            for (int j = 0; j < NV; ++j)
                s[j] = base[j];
        } else if constexpr (TREE) {
            if (d != dprev + 1) {
                if (LEVELS == kMaxDepth - 1 || d - 1 <= LEVELS) {
#pragma unroll
                    for (int j = 0; j < NV; ++j)
                        s[j] = *reinterpret_cast<const float4*>(parent_base + d * kLevelBytes + j * 256 * 16);
                } else {
                    // Replay the ancestors of depths LEVELS + 1 .. d - 1, each
                    // the latest position before this one with its depth.
#pragma unroll
                    for (int j = 0; j < NV; ++j)
                        s[j] = sm.stack[LEVELS - 1][j][tid];
                    for (int e = LEVELS + 1; e < d; ++e) {
                        const uint64_t m = __builtin_amdgcn_ballot_w64(c.dep_l == e) & ((1ull << it) - 1);
                        NodeOps<D> anc;
                        c.load_node(anc, 63 - __builtin_clzll(m));
                        (void)node_update<D>(s, anc);
                    }
                }
            }
        }
        const float out = node_update<D>(s, ring[p]);
        c.store_o(it, out);
        if constexpr (TREE) {
            if (d <= LEVELS) {
#pragma unroll
                for (int j = 0; j < NV; ++j)
                    *reinterpret_cast<float4*>(save_base + d * kLevelBytes + j * 256 * 16) = s[j];
            }
        }
        dprev = d;
        if (it + RING < kMaxNodes)
            c.load_node(ring[p], it + RING);
        // A chain walk has no branches, so without this the scheduler would
        // sink each refill next to its use and the ring would prefetch nothing.
        if constexpr (!TREE)
            __builtin_amdgcn_sched_barrier(0);
        return true;
    };
    walk_all(step, std::make_integer_sequence<int, kMaxNodes>{});
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

// The prep launch (tables and node operands) of a tree, or of a block when
// parent is null.
template <int D, typename Act>
static void launch_prep(const Geo& g, int n, const void* tail, const void* w, const int32_t* parent, const void* x,
                        const float* a, const float* b, const TreeWs& W, int32_t* status, hipStream_t s) {
    const int64_t node_wgs = static_cast<int64_t>(g.B) * n * g.Hk;
    auto grid = [&](int npw) { return dim3(static_cast<unsigned>(g.B + g.B * g.Hk * ((n + npw - 1) / npw))); };
    if (node_wgs > 8 * 256)   // more than eight node workgroups per CU
        hipLaunchKernelGGL((tree_prep_kernel<D, Act, 4>), grid(4), dim3(256), 0, s, static_cast<const Act*>(tail),
                           static_cast<const Act*>(w), n, parent, static_cast<const Act*>(x), a, b, W, status, g.B,
                           g.Hk, g.Hv, g.C);
    else
        hipLaunchKernelGGL((tree_prep_kernel<D, Act, 1>), grid(1), dim3(256), 0, s, static_cast<const Act*>(tail),
                           static_cast<const Act*>(w), n, parent, static_cast<const Act*>(x), a, b, W, status, g.B,
                           g.Hk, g.Hv, g.C);
}

hipError_t launch_tree_verify(const Geo& g, const float* S, const void* tail, const void* w, int n,
                              const int32_t* parent, const void* x, const float* a, const float* b, float* o,
                              int32_t* status, void* ws, hipStream_t s) {
    const TreeWs W = tree_ws_carve(ws, g.B, n, g.Hk, g.Hv, g.D);
    hipError_t e = dispatch(g, [&](auto dtag, auto atag) {
        constexpr int D = decltype(dtag)::value;
        using Act = decltype(atag);
        launch_prep<D, Act>(g, n, tail, w, parent, x, a, b, W, status, s);
    });
    if (e != hipSuccess)
        return e;
    return dispatch(g, [&](auto dtag, auto) {
        constexpr int D = decltype(dtag)::value;
        const int bph = D / (4 * Row<D>::RPW);
        const unsigned grid = static_cast<unsigned>(g.B * g.Hv * bph);
        // More workgroups than two per CU: the form for several trees per CU.
        if (grid > 2u * 256u)
            hipLaunchKernelGGL((tree_verify_kernel<D, WalkWide, WalkKind::Tree>), dim3(grid), dim3(256), 0, s, S, n,
                               W, o, g.Hk, g.Hv, bph);
        else
            hipLaunchKernelGGL((tree_verify_kernel<D, WalkDeep, WalkKind::Tree>), dim3(grid), dim3(256), 0, s, S, n,
                               W, o, g.Hk, g.Hv, bph);
    });
}

// ------------------------------------------------------------ tree verify, UT form
//
// The same outputs as the walk, reached without building any node's state:
// the tree counterpart of the chunked (WY/UT) form, with "ancestor of" in
// place of "earlier in the chunk".  Per (sequence, value head), with the
// nodes in index order (every parent before its children), j <= i meaning
// "j is i or an ancestor of i", rho(i, j) the product of the gates alpha on
// the path (j, i] and gamma_i the product over the whole path to i:
//   S_i = gamma_i S_c + sum_{j <= i} rho(i, j) u_j k_j^T
//   u_j = beta_j (v_j - gamma_j S_c k_j - sum_{l < j} rho(j, l) (k_l.k_j) u_l)
// so (I + A) U = diag(beta) (V - diag(gamma) K S_c^T) with
// A[j][l] = beta_j rho(j, l) (k_j.k_l) over strict ancestors l, and
//   o_i = s (S_c q_i gamma_i + sum_{j <= i} rho(i, j) (q_i.k_j) u_j).
// With M[i][j] = rho(i, j) (q_i.k_j) and R = M (I + A)^-1 diag(beta):
//   o_i = s (S_c e_i + sum_l R[i][l] v_l),   e_i = gamma_i q_i - sum_l R[i][l] gamma_l k_l.
// Every matrix above is 32 x 32 or 32 x 128, and the checkpoint enters once,
// as the product E S_c^T: each head's checkpoint is read once and nothing is
// written but the outputs.  The Gram matrices, E, R V and E S_c^T run on
// bf16 MFMA (16x16x32) with both operands split into two bf16 parts (x = hi
// + lo; three products, about 16 significant bits each way); the
// off-diagonal block of (I + A)^-1 and R on fp32 MFMA (16x16x4); the
// diagonal 16 x 16 blocks of (I + A)^-1 by substitution.
// The arithmetic is reordered against token-by-token decode, so the outputs
// agree with it to rounding, not bit for bit.
//
// One workgroup per (sequence, value head), four waves, and no other launch:
// the workgroup convolves the raw inputs of its q/k head's and its value
// head's channels itself.  Every node's window lies on the node's own path,
// so the workgroup stages the raw inputs of all its nodes and the four tail
// entries as rows of one LDS table and convolves each node from the rows of
// itself and its nearest ancestors.  Each wave's share of the checkpoint
// (D / 4 rows; for D = 32, 16 rows shared by two waves) is loaded right after
// the raw inputs, in the operand layout of the final product, and stays in
// flight through the convolution and the small matrices.
template <int D, typename Act>
struct alignas(16) UtSmem {
    static constexpr int P = D + 4;           // bf16 row of D plus 8 bytes: a quarter-wave's reads hit distinct banks
    static constexpr int PS = kMaxNodes + 4;  // 16-byte aligned rows of the 32 x 32 matrices
    static constexpr int NCH = 3 * D;         // the q | k | v channels the workgroup convolves
    static constexpr int XR = kMaxNodes + 4;  // staging rows: the nodes' raw inputs, then tail entries 0..3
    union {
        struct {                              // raw conv inputs, until every thread holds its outputs
            Act x[XR][NCH];
            Act w[NCH][4];
        };
        struct {                              // then the split operands
            __bf16 kh[kMaxNodes][P], kl[kMaxNodes][P];   // k = kh + kl, each part rounded to bf16
            __bf16 qh[kMaxNodes][P], ql[kMaxNodes][P];   // q, then e
        };
    };
    // Each 32 x 32 buffer holds two matrices whose lifetimes are separated by
    // a barrier, so that three workgroups fit in a CU's LDS (bf16 inputs).
    union {
        float rho[kMaxNodes][PS];   // until A and M are formed
        float t[kMaxNodes][PS];     // (I + A)^-1, after
    };
    union {
        float ga[kMaxNodes][PS];    // A, until (I + A)^-1 is complete
        float r[kMaxNodes][PS];     // R, after
    };
    float gm[kMaxNodes][PS];   // M
    float rg[kMaxNodes][PS];   // R diag(gamma)
    float al[kMaxNodes], be[kMaxNodes], gam[kMaxNodes];
    int32_t par[kMaxNodes];
    int32_t src[kMaxNodes][4];   // staging rows of each node's conv window, oldest first
    int32_t ok;
};

using ut_f4 = __attribute__((ext_vector_type(4))) float;
using ut_bf4 = __attribute__((ext_vector_type(4))) __bf16;
using ut_bf8 = __attribute__((ext_vector_type(8))) __bf16;

// x = hi + lo with hi the bf16 rounding of x and lo that of the remainder.
__device__ __forceinline__ void ut_split(float x, __bf16& hi, __bf16& lo) {
    hi = static_cast<__bf16>(x);
    lo = static_cast<__bf16>(x - static_cast<float>(hi));
}
template <typename V>
__device__ __forceinline__ void ut_split_at(float x, V& hi, V& lo, int e) {
    const __bf16 h = static_cast<__bf16>(x);
    hi[e] = h;
    lo[e] = static_cast<__bf16>(x - static_cast<float>(h));
}
__device__ __forceinline__ ut_bf8 ut_cat(const __bf16* p0, const __bf16* p1) {
    return __builtin_shufflevector(*reinterpret_cast<const ut_bf4*>(p0), *reinterpret_cast<const ut_bf4*>(p1), 0, 1,
                                   2, 3, 4, 5, 6, 7);
}
// The three-product bf16 MFMA of split operands: a.b to about 16 bits each way.
__device__ __forceinline__ ut_f4 ut_mma3(ut_bf8 ah, ut_bf8 al, ut_bf8 bh, ut_bf8 bl, ut_f4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
}

// SiLU of the 4-tap conv of bf16 inputs: taps (oldest, next) packed in x01 and
// (next, newest) in x23, the channel's taps in w (.x = taps 0, 1; .y = 2, 3),
// summed by the bf16 dot product into fp32; SiLU as in conv_silu.
__device__ __forceinline__ float ut_conv_bf16(uint2 w, uint32_t x01, uint32_t x23) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf2;
    float z = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, w.x), __builtin_bit_cast(bf2, x01), 0.0f,
                                              false);
    z = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, w.y), __builtin_bit_cast(bf2, x23), z, false);
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

// Global channel of the workgroup's local channel lc: q of its q/k head, then
// k, then v of its value head.
template <int D>
__device__ __forceinline__ int ut_channel(int lc, int g, int h, int Hk) {
    return lc < D ? g * D + lc : lc < 2 * D ? Hk * D + g * D + (lc - D) : 2 * Hk * D + h * D + (lc - 2 * D);
}

// Two workgroups per CU: the checkpoint rows in flight (64 registers), the
// conv operands and the split products need about 194 registers, and a
// budget of 168 (three per CU) spills.  Measured on the 27B-class layer, 64
// trees: 88.8 us at two per CU against 113.7 at three (31 registers spilled).
// With SPLIT = 2 each wave holds half as many checkpoint rows (133 registers).
// SPLIT = 2 (small batches, D = 128): two workgroups per (sequence, value
// head), each with half the rows: its share of the checkpoint, of the value
// convolution and of the last product; both build the small matrices.
template <int D, typename Act, int SPLIT = 1>
__device__ __forceinline__ void tree_ut_body(int bid, int nblocks,
    const float* __restrict__ Sc, const Act* __restrict__ tail, const Act* __restrict__ w, int n,
    const int32_t* __restrict__ parent, const Act* __restrict__ x, const float* __restrict__ a,
    const float* __restrict__ b, float* __restrict__ o, int32_t* __restrict__ status, int Hk, int Hv, int C) {
    static_assert(D == 32 || D == 128, "head dims 32 and 128");
    using f4 = ut_f4;
    using bf8 = ut_bf8;
    using Sm = UtSmem<D, Act>;
    constexpr int NT = kMaxNodes;                 // nodes padded to two tiles of 16
    static_assert(SPLIT == 1 || (SPLIT == 2 && D == 128), "rows split in two for D = 128 only");
    constexpr int RT = D >= 64 ? D / 64 / SPLIT : 1;   // row tiles of 16 per wave in the last product
    constexpr int NTW = D >= 64 ? 2 : 1;          // node tiles per wave in the last product
    constexpr int KS = D / 16;                    // 16-wide blocks of the key dim
    constexpr int ET = D / 32;                    // tiles of e per wave
    constexpr int NCH = Sm::NCH;
    constexpr int VPL = 16 / sizeof(Act);         // inputs per 16-byte load
    constexpr int LPN = NCH / VPL;                // 16-byte loads per node row
    constexpr int XL = (NT * LPN + 255) / 256;    // per thread
    constexpr int TL = (NCH + 255) / 256;         // tail and weight quads per thread
    constexpr int CPS = D / 8;                    // q (and k) channels per thread in the conv
    __shared__ Sm sm;

    // The index arithmetic is made to depend on every argument, so all the
    // argument loads issue together (one kernel-argument round trip).
    asm volatile("" : "+s"(Hv) : "s"(Sc), "s"(tail), "s"(w), "s"(n), "s"(parent), "s"(x), "s"(a), "s"(b), "s"(o),
                 "s"(status), "s"(Hk), "s"(C));
    const int idp = xcd_packed_id(bid, nblocks);
    const int id = idp / SPLIT, half = idp % SPLIT;   // a head's two halves share an XCD
    const int bq = id / Hv, h = id % Hv, g = h / (Hv / Hk);
    const int m0 = bq * n;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int q = lane >> 4, c = lane & 15;
    const int rb = D >= 64 ? half * (D / SPLIT) + wave * 16 * RT : 16 * (wave >> 1);   // first checkpoint row of this wave
    const int u0 = D >= 64 ? 0 : (wave & 1);                      // first node tile of this wave

    // Loads, all unconditional: the raw inputs of every node (padding nodes
    // read node n - 1 and are zeroed after), the tail and the taps, the parent
    // row and the gates first; then this wave's checkpoint rows, which stay in
    // flight through the convolution and the small matrices.
    using Q = Quad<Act>;
    f4 xr[XL];
#pragma unroll
    for (int e = 0; e < XL; ++e) {
        const int idx = min(tid + 256 * e, NT * LPN - 1), node = min(idx / LPN, n - 1), f = idx % LPN;
        const int lc = f * VPL;
        xr[e] = *reinterpret_cast<const f4*>(x + static_cast<size_t>(m0 + node) * C + ut_channel<D>(lc, g, h, Hk));
    }
    typename Q::raw tr[TL], wr[TL];
#pragma unroll
    for (int e = 0; e < TL; ++e) {
        const int lc = min(tid + 256 * e, NCH - 1), gc = ut_channel<D>(lc, g, h, Hk);
        tr[e] = Q::load(tail + (static_cast<size_t>(bq) * C + gc) * 4);
        wr[e] = Q::load(w + static_cast<size_t>(gc) * 4);
    }
    const int gn = min(lane & (NT - 1), n - 1);
    const float a_in = a[static_cast<size_t>(m0 + gn) * Hv + h];
    const float b_in = b[static_cast<size_t>(m0 + gn) * Hv + h];
    const int32_t pa_in = parent ? parent[m0 + gn] : gn - 1;

    // This wave's checkpoint rows, in the B-operand layout of the last product:
    // they arrive while the small matrices are built.
    const float* Sh = Sc + (static_cast<size_t>(bq) * Hv + h) * D * D;
    f4 sv[RT][KS];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int k = 0; k < KS; ++k)
            sv[t][k] = __builtin_nontemporal_load(
                reinterpret_cast<const f4*>(Sh + static_cast<size_t>(rb + 16 * t + c) * D + 16 * k + 4 * q));

    // Stage the raw inputs: node rows as loaded, the tail turned into four
    // rows (entry 0, the oldest, first), the taps as they are.
#pragma unroll
    for (int e = 0; e < XL; ++e) {
        const int idx = tid + 256 * e;
        if (NT * LPN % 256 == 0 || idx < NT * LPN)
            *reinterpret_cast<f4*>(&sm.x[idx / LPN][(idx % LPN) * VPL]) = xr[e];
    }
#pragma unroll
    for (int e = 0; e < TL; ++e) {
        const int lc = tid + 256 * e;
        if (NCH % 256 == 0 || lc < NCH) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sm.x[NT + j][lc] = Q::elem(tr[e], j);
            Q::store(&sm.w[lc][0], wr[e]);
        }
    }
    // Wave 0, lane i < n: node i's gates, its depth and nearest ancestors, the
    // check of the parent row (parent[0] == -1, 0 <= parent[i] < i, depth <=
    // 8; a block is a chain and always valid), the staging rows of its
    // window, and rho and gamma: lane i clears row i of rho and walks up from
    // node i (the gates and parents it reads were written by lanes of the same
    // wave, whose LDS accesses are processed in order).
    if (wave == 0) {
        const bool live = lane < n;
        int ok = 1, depth = 0, anc[3] = {-1, -1, -1};
        if (parent == nullptr) {
            depth = lane + 1;
#pragma unroll
            for (int k = 0; k < 3; ++k)
                anc[k] = lane - 1 - k;
        } else {
            const int p = live ? pa_in : -1;
            const bool bad = live && (lane == 0 ? p != -1 : (p < 0 || p >= lane));
            if (__any(bad)) {
                ok = 0;
            } else {
                int cur = live ? lane : -1;
#pragma unroll
                for (int st = 0; st <= kMaxDepth; ++st) {
                    depth += cur >= 0 ? 1 : 0;
                    const int up = __shfl(p, cur >= 0 ? cur : 0, kWave);
                    if (st < 3)
                        anc[st] = cur >= 0 ? up : -1;
                    cur = cur >= 0 ? up : -1;
                }
                ok = __any(live && cur >= 0) ? 0 : 1;
            }
        }
        if (lane < NT) {
            int src[4] = {0, 0, 0, 0};
            if (ok && live) {
                src[3] = lane;
#pragma unroll
                for (int k = 1; k <= 3; ++k)
                    src[3 - k] = k <= depth - 1 ? anc[k - 1] : NT + 3 + depth - k;
            }
#pragma unroll
            for (int k = 0; k < 4; ++k)
                sm.src[lane][k] = src[k];
            float al_v, be_v;
            gates(a_in, b_in, al_v, be_v);
            sm.al[lane] = live ? al_v : 1.0f;
            sm.be[lane] = live ? be_v : 0.0f;
            sm.par[lane] = live && ok ? pa_in : -1;
#pragma unroll
            for (int l = 0; l < NT; l += 4)
                *reinterpret_cast<f4*>(&sm.rho[lane][l]) = f4{0.0f, 0.0f, 0.0f, 0.0f};
            float prod = 1.0f;
            if (parent == nullptr) {
                if (lane >= n)
                    sm.rho[lane][lane] = 1.0f;
                for (int l = live ? lane : -1; l >= 0; --l) {
                    sm.rho[lane][l] = prod;
                    prod *= sm.al[l];
                }
            } else {
                int cur = lane;
                for (int st = 0; st < NT && cur >= 0 && cur < NT; ++st) {
                    sm.rho[lane][cur] = prod;
                    prod *= sm.al[cur];
                    cur = sm.par[cur];
                }
            }
            sm.gam[lane] = prod;
        }
        if (lane == 0)
            sm.ok = ok;
    }
    __syncthreads();
    if (!sm.ok) {   // malformed tree: reported, nothing written
        if (status && h == 0 && half == 0 && tid == 0)
            status[bq] = 5;
        return;
    }
    if (status && h == 0 && half == 0 && tid == 0)
        status[bq] = 0;

    // The conv.  q and k: thread (node tid / 8, part tid % 8) convolves CPS
    // channels of each, and the eight threads of a node reduce its norms.  v:
    // every lane convolves the values of the final product's B operand it
    // holds: slot e of lane (q, c) is node 4 q + e, or 16 + 4 q + e - 4, at
    // rows rb + 16 t + c.  bf16 inputs: each tap pair (oldest two, newest two)
    // of a channel is packed into one word and summed against the packed taps
    // by the bf16 dot product, with no widening (a third of the conv's
    // instructions); a padding node's window reads valid rows and its outputs
    // are zeroed by a mask.
    float qn[CPS], kn[CPS];
    float vv[RT][8];
    if constexpr (sizeof(Act) == 2) {
        const uint32_t* xw = reinterpret_cast<const uint32_t*>(&sm.x[0][0]);   // two channels per word
        const uint2* ww = reinterpret_cast<const uint2*>(&sm.w[0][0]);          // one channel's taps per uint2
        {
            const int node = tid >> 3, part = tid & 7;
            const int4 sr = *reinterpret_cast<const int4*>(&sm.src[node][0]);
            const int so[4] = {sr.x * (NCH / 2), sr.y * (NCH / 2), sr.z * (NCH / 2), sr.w * (NCH / 2)};
            const float mask = node < n ? 1.0f : 0.0f;
            float sq = 0.0f, sk = 0.0f;
#pragma unroll
            for (int seg = 0; seg < 2; ++seg) {
#pragma unroll
                for (int i = 0; i < CPS / 2; ++i) {
                    const int wo = seg * (D / 2) + part * (CPS / 2) + i;
                    uint32_t r[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        r[k] = xw[so[k] + wo];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const uint32_t sel = hh ? 0x07060302u : 0x05040100u;
                        const uint2 wv = ww[seg * D + part * CPS + 2 * i + hh];
                        const float y = ut_conv_bf16(wv, __builtin_amdgcn_perm(r[1], r[0], sel),
                                                     __builtin_amdgcn_perm(r[3], r[2], sel)) * mask;
                        if (seg == 0) {
                            qn[2 * i + hh] = y;
                            sq = __builtin_fmaf(y, y, sq);
                        } else {
                            kn[2 * i + hh] = y;
                            sk = __builtin_fmaf(y, y, sk);
                        }
                    }
                }
            }
            sq = group_sum<8>(sq);
            sk = group_sum<8>(sk);
            const float rq = __builtin_amdgcn_rsqf(sq + kEps), rk = __builtin_amdgcn_rsqf(sk + kEps);
#pragma unroll
            for (int j = 0; j < CPS; ++j) {
                qn[j] *= rq;
                kn[j] *= rk;
            }
        }
        const uint16_t* xh = reinterpret_cast<const uint16_t*>(&sm.x[0][0]);
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const int lc = 2 * D + rb + 16 * t + c;
            const uint2 wv = ww[lc];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int node = e < 4 ? 4 * q + e : 12 + 4 * q + e;
                const int4 sr = *reinterpret_cast<const int4*>(&sm.src[node][0]);
                const uint32_t x01 = xh[sr.x * NCH + lc] | (static_cast<uint32_t>(xh[sr.y * NCH + lc]) << 16);
                const uint32_t x23 = xh[sr.z * NCH + lc] | (static_cast<uint32_t>(xh[sr.w * NCH + lc]) << 16);
                vv[t][e] = ut_conv_bf16(wv, x01, x23) * (node < n ? 1.0f : 0.0f);
            }
        }
    } else {
        {
            const int node = tid >> 3, part = tid & 7;
            int srow[4];
    #pragma unroll
            for (int k = 0; k < 4; ++k)
                srow[k] = sm.src[node][k];
            float sq = 0.0f, sk = 0.0f;
    #pragma unroll
            for (int j4 = 0; j4 < CPS; j4 += 4) {
                const int l0 = part * CPS + j4;
                float xq[4][4], xk[4][4];   // [tap][channel]
    #pragma unroll
                for (int k = 0; k < 4; ++k) {
                    Q::to_float(Q::load(&sm.x[srow[k]][l0]), xq[k]);
                    Q::to_float(Q::load(&sm.x[srow[k]][D + l0]), xk[k]);
                }
    #pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    float wf[4], win[4];
                    Q::to_float(Q::load(&sm.w[l0 + jj][0]), wf);
    #pragma unroll
                    for (int k = 0; k < 4; ++k)
                        win[k] = xq[k][jj];
                    const float yq = node < n ? conv_silu(wf, win) : 0.0f;
                    Q::to_float(Q::load(&sm.w[D + l0 + jj][0]), wf);
    #pragma unroll
                    for (int k = 0; k < 4; ++k)
                        win[k] = xk[k][jj];
                    const float yk = node < n ? conv_silu(wf, win) : 0.0f;
                    qn[j4 + jj] = yq;
                    kn[j4 + jj] = yk;
                    sq = __builtin_fmaf(yq, yq, sq);
                    sk = __builtin_fmaf(yk, yk, sk);
                }
            }
            sq = group_sum<8>(sq);
            sk = group_sum<8>(sk);
            const float rq = __builtin_amdgcn_rsqf(sq + kEps), rk = __builtin_amdgcn_rsqf(sk + kEps);
    #pragma unroll
            for (int j = 0; j < CPS; ++j) {
                qn[j] *= rq;
                kn[j] *= rk;
            }
        }
    #pragma unroll
        for (int t = 0; t < RT; ++t) {
            const int lc = 2 * D + rb + 16 * t + c;
            float wf[4];
            Q::to_float(Q::load(&sm.w[lc][0]), wf);
    #pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int node = e < 4 ? 4 * q + e : 12 + 4 * q + e;
                float win[4];
    #pragma unroll
                for (int k = 0; k < 4; ++k)
                    win[k] = widen(sm.x[sm.src[node][k]][lc]);
                vv[t][e] = node < n ? conv_silu(wf, win) : 0.0f;
            }
        }
    }
    __syncthreads();   // the staged inputs are dead: the split operands take their place
    {
        const int node = tid >> 3, part = tid & 7;
#pragma unroll
        for (int j0 = 0; j0 < CPS; j0 += 4) {
            ut_bf4 hi, lo;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ut_split_at(qn[j0 + j], hi, lo, j);
            *reinterpret_cast<ut_bf4*>(&sm.qh[node][part * CPS + j0]) = hi;
            *reinterpret_cast<ut_bf4*>(&sm.ql[node][part * CPS + j0]) = lo;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ut_split_at(kn[j0 + j], hi, lo, j);
            *reinterpret_cast<ut_bf4*>(&sm.kh[node][part * CPS + j0]) = hi;
            *reinterpret_cast<ut_bf4*>(&sm.kl[node][part * CPS + j0]) = lo;
        }
    }
    __syncthreads();

    // Every wave takes one 16x16 tile (I, J) of K K^T and of Q K^T, and forms
    // A and M on it from the gates on the ancestor paths (rho is 0 off them).
    // Tile (0, 1) lies above the diagonal, where neither has an entry.
    {
        const int I = wave >> 1, J = wave & 1;
        f4 gk0 = {0.0f, 0.0f, 0.0f, 0.0f}, gk1 = gk0, gq0 = gk0, gq1 = gk0;
        if (!(I == 0 && J == 1)) {
#pragma unroll
            for (int m = 0; m < KS / 2; ++m) {
                const int c0 = 32 * m + 4 * q, c1 = c0 + 16;
                const bf8 akh = ut_cat(&sm.kh[16 * I + c][c0], &sm.kh[16 * I + c][c1]);
                const bf8 akl = ut_cat(&sm.kl[16 * I + c][c0], &sm.kl[16 * I + c][c1]);
                const bf8 aqh = ut_cat(&sm.qh[16 * I + c][c0], &sm.qh[16 * I + c][c1]);
                const bf8 aql = ut_cat(&sm.ql[16 * I + c][c0], &sm.ql[16 * I + c][c1]);
                const bf8 bkh = ut_cat(&sm.kh[16 * J + c][c0], &sm.kh[16 * J + c][c1]);
                const bf8 bkl = ut_cat(&sm.kl[16 * J + c][c0], &sm.kl[16 * J + c][c1]);
                gk0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(akh, bkh, gk0, 0, 0, 0);
                gq0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aqh, bkh, gq0, 0, 0, 0);
                gk1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(akh, bkl, gk1, 0, 0, 0);
                gq1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aqh, bkl, gq1, 0, 0, 0);
                gk1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(akl, bkh, gk1, 0, 0, 0);
                gq1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aql, bkh, gq1, 0, 0, 0);
            }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = 16 * I + 4 * q + v, l = 16 * J + c;
            const float r = sm.rho[i][l];
            sm.ga[i][l] = l == i ? 0.0f : sm.be[i] * r * (gk0[v] + gk1[v]);
            sm.gm[i][l] = r * (gq0[v] + gq1[v]);
        }
    }
    __syncthreads();

    // (I + A)^-1: the two diagonal 16x16 blocks by substitution (wave 0, lane =
    // (block, column)); the block above the diagonal is 0.
    if (wave == 0 && lane < NT) {
        const int b0 = 16 * (lane >> 4), j = lane & 15;
        float X[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float arow[16];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const f4 a4 = *reinterpret_cast<const f4*>(&sm.ga[b0 + i][b0 + 4 * p]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    arow[4 * p + e] = a4[e];
            }
            float s = i == j ? 1.0f : 0.0f;
#pragma unroll
            for (int k = 0; k < i; ++k)
                s = __builtin_fmaf(-arow[k], X[k], s);
            X[i] = s;
            sm.t[b0 + i][b0 + j] = s;
        }
    } else if (wave == 1) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
            sm.t[4 * q + v][16 + c] = 0.0f;
    }
    __syncthreads();
    // the block below it: T_10 = -T_11 (A_10 T_00)
    if (wave == 0) {
        f4 z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
            z = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.ga[16 + c][4 * q + s], sm.t[4 * q + s][c], z, 0, 0, 0);
        f4 tt = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
            tt = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.t[16 + c][16 + 4 * q + s], z[s], tt, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v)
            sm.t[16 + 4 * q + v][c] = -tt[v];
    }
    __syncthreads();

    // R = M (I + A)^-1 diag(beta) and R diag(gamma), one 16x16 tile per wave.
    {
        const int I = wave >> 1, J = wave & 1;
        f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if (!(I == 0 && J == 1)) {
#pragma unroll
            for (int K = 0; K < 2; ++K)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.gm[16 * I + c][16 * K + 4 * q + s],
                                                               sm.t[16 * K + 4 * q + s][16 * J + c], acc, 0, 0, 0);
        }
        const float bc = sm.be[16 * J + c], gc = sm.gam[16 * J + c];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float rv = acc[v] * bc;
            sm.r[16 * I + 4 * q + v][16 * J + c] = rv;
            sm.rg[16 * I + 4 * q + v][16 * J + c] = rv * gc;
        }
    }
    __syncthreads();

    // e = gamma q - (R diag(gamma)) K, written over q; and the accumulators of
    // the last product start at R V.  Both on split bf16 MFMA with the 32
    // nodes as k: slot e of lane (q, c) is node 4 q + e, or 16 + 4 q + e - 4.
    auto row_split = [&](const float (*M)[Sm::PS], int row, bf8& hi, bf8& lo) {
        const f4 x0 = *reinterpret_cast<const f4*>(&M[row][4 * q]);
        const f4 x1 = *reinterpret_cast<const f4*>(&M[row][16 + 4 * q]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ut_split_at(x0[e], hi, lo, e);
            ut_split_at(x1[e], hi, lo, 4 + e);
        }
    };
#pragma unroll
    for (int e = 0; e < ET; ++e) {
        const int tau = wave * ET + e, U = tau & 1, Ct = tau >> 1, col = 16 * Ct + c;
        bf8 ah, al;
        row_split(sm.rg, 16 * U + c, ah, al);
        bf8 bh, bl;   // k of the slot nodes, one column: 2-byte reads down the rows
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int l = e < 4 ? 4 * q + e : 12 + 4 * q + e;
            bh[e] = sm.kh[l][col];
            bl[e] = sm.kl[l][col];
        }
        const f4 z = ut_mma3(ah, al, bh, bl, f4{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = 16 * U + 4 * q + v;
            const float qv = static_cast<float>(sm.qh[i][col]) + static_cast<float>(sm.ql[i][col]);
            ut_split(sm.gam[i] * qv - z[v], sm.qh[i][col], sm.ql[i][col]);
        }
    }
    f4 acc[RT][NTW];
#pragma unroll
    for (int u = 0; u < NTW; ++u) {
        bf8 ah, al;
        row_split(sm.r, 16 * (u0 + u) + c, ah, al);
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            bf8 vh, vl;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                ut_split_at(vv[t][e], vh, vl, e);
            acc[t][u] = ut_mma3(ah, al, vh, vl, f4{0.0f, 0.0f, 0.0f, 0.0f});
        }
    }
    __syncthreads();

    // o = s (E S_c^T + R V) over this wave's rows, E and the checkpoint rows
    // split alike.  Lane (q, c) holds, for k-step m, the columns 32 m + 4 q +
    // 0..3 and 32 m + 16 + 4 q + 0..3 of its row, in both operands.
#pragma unroll
    for (int m = 0; m < KS / 2; ++m) {
        bf8 shi[RT], slo[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                ut_split_at(sv[t][2 * m + e / 4][e % 4], shi[t], slo[t], e);
#pragma unroll
        for (int u = 0; u < NTW; ++u) {
            const int row = 16 * (u0 + u) + c, c0 = 32 * m + 4 * q;
            const bf8 ah = ut_cat(&sm.qh[row][c0], &sm.qh[row][c0 + 16]);
            const bf8 al = ut_cat(&sm.ql[row][c0], &sm.ql[row][c0 + 16]);
#pragma unroll
            for (int t = 0; t < RT; ++t)
                acc[t][u] = ut_mma3(ah, al, shi[t], slo[t], acc[t][u]);
        }
    }
#pragma unroll
    for (int u = 0; u < NTW; ++u)
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int node = 16 * (u0 + u) + 4 * q + v;
                if (node < n)
                    o[(static_cast<size_t>(m0 + node) * Hv + h) * D + rb + 16 * t + c] = Scale<D>::value * acc[t][u][v];
            }
}

template <int D, typename Act, int SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void tree_ut_kernel(
    const float* __restrict__ Sc, const Act* __restrict__ tail, const Act* __restrict__ w, int n,
    const int32_t* __restrict__ parent, const Act* __restrict__ x, const float* __restrict__ a,
    const float* __restrict__ b, float* __restrict__ o, int32_t* __restrict__ status, int Hk, int Hv, int C) {
    tree_ut_body<D, Act, SPLIT>(blockIdx.x, gridDim.x, Sc, tail, w, n, parent, x, a, b, o, status, Hk, Hv, C);
}

// The one-launch UT verify and the prep of a workspace for a prepared commit,
// in one grid: workgroups [0, ut_blocks) verify (their ids packed by XCD as
// in tree_ut_kernel), the rest are tree_prep_kernel's workgroups.  The two
// parts share nothing but the inputs, so at small batches (where neither
// fills the chip) they run side by side instead of one after the other.
// The tree's status is written by the verify part only.
template <int D, typename Act, int SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void tree_ut_prep_kernel(
    const float* __restrict__ Sc, const Act* __restrict__ tail, const Act* __restrict__ w, int n,
    const int32_t* __restrict__ parent, const Act* __restrict__ x, const float* __restrict__ a,
    const float* __restrict__ b, float* __restrict__ o, int32_t* __restrict__ status, TreeWs ws, int B, int Hk,
    int Hv, int C, int ut_blocks) {
    if (static_cast<int>(blockIdx.x) < ut_blocks)
        tree_ut_body<D, Act, SPLIT>(blockIdx.x, ut_blocks, Sc, tail, w, n, parent, x, a, b, o, status, Hk, Hv, C);
    else
        tree_prep_body<D, Act, 1>(blockIdx.x - ut_blocks, tail, w, n, parent, x, a, b, ws, nullptr, B, Hk, Hv, C);
}

// The two-launch form of the same verify: the prep launch convolves and
// normalises every node's operands into the workspace (where a prepared
// commit can read them), spread over many workgroups, and the UT workgroup
// reads them from there.
template <int D>
struct UtWsSmem {
    static constexpr int P = D + 4;           // bf16 row of D plus 8 bytes: a quarter-wave's reads hit distinct banks
    static constexpr int PS = kMaxNodes + 4;  // 16-byte aligned rows of the 32 x 32 matrices
    __bf16 kh[kMaxNodes][P], kl[kMaxNodes][P];   // k = kh + kl, each part rounded to bf16
    __bf16 qh[kMaxNodes][P], ql[kMaxNodes][P];   // q, then e
    // Each 32 x 32 buffer holds two matrices whose lifetimes are separated by
    // a barrier, so that three workgroups fit in a CU's LDS.
    union {
        float rho[kMaxNodes][PS];   // until A and M are formed
        float t[kMaxNodes][PS];     // (I + A)^-1, after
    };
    union {
        float ga[kMaxNodes][PS];    // A, until (I + A)^-1 is complete
        float r[kMaxNodes][PS];     // R, after
    };
    float gm[kMaxNodes][PS];   // M
    float rg[kMaxNodes][PS];   // R diag(gamma)
    float al[kMaxNodes], be[kMaxNodes], gam[kMaxNodes];
    int32_t par[kMaxNodes];
};

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void tree_ut_ws_kernel(const float* __restrict__ Sc, int n,
                                                      const int32_t* __restrict__ parent, TreeWs ws,
                                                      float* __restrict__ o, int Hk, int Hv) {
    static_assert(D == 32 || D == 128, "head dims 32 and 128");
    using f4 = ut_f4;
    using bf8 = ut_bf8;
    constexpr int NT = kMaxNodes;                 // nodes padded to two tiles of 16
    constexpr int RT = D >= 64 ? D / 64 : 1;      // row tiles of 16 per wave in the last product
    constexpr int NTW = D >= 64 ? 2 : 1;          // node tiles per wave in the last product
    constexpr int KS = D / 16;                    // 16-wide blocks of the key dim
    constexpr int ET = D / 32;                    // tiles of e per wave
    __shared__ UtWsSmem<D> sm;

    // The index arithmetic is made to depend on every argument, so all the
    // argument loads issue together (one kernel-argument round trip).
    asm volatile("" : "+s"(Hv) : "s"(Sc), "s"(n), "s"(parent), "s"(ws.qk), "s"(ws.v), "s"(ws.abk), "s"(ws.tab), "s"(o),
                 "s"(Hk));
    const int id = xcd_packed_id(blockIdx.x, gridDim.x);
    const int bq = id / Hv, h = id % Hv, g = h / (Hv / Hk);
    const int m0 = bq * n;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int q = lane >> 4, c = lane & 15;
    const int rb = D >= 64 ? wave * 16 * RT : 16 * (wave >> 1);   // first checkpoint row of this wave
    const int u0 = D >= 64 ? 0 : (wave & 1);                      // first node tile of this wave

    // Loads, all unconditional (padding nodes read node n - 1 and are zeroed
    // after): q and k of the q/k head and the gates first, then this wave's
    // checkpoint rows and values, which stay in flight through the small
    // matrices.
    constexpr int QK4 = NT * D / 2 / 256;   // float4 of q|k per thread
    f4 qk[QK4];
#pragma unroll
    for (int e = 0; e < QK4; ++e) {
        const int idx = tid + 256 * e, node = min(idx / (D / 2), n - 1), f = idx % (D / 2);
        qk[e] = *reinterpret_cast<const f4*>(ws.qk + (static_cast<size_t>(m0 + node) * Hk + g) * 2 * D + 4 * f);
    }
    const int gn = min(lane & (NT - 1), n - 1);
    const float al_in = ws.abk[(static_cast<size_t>(m0 + gn) * Hv + h) * 4];
    const float be_in = ws.abk[(static_cast<size_t>(m0 + gn) * Hv + h) * 4 + 1];
    // (a block has no parent array: read some valid word, keep gn - 1)
    const int32_t pa_raw = *(parent ? parent + m0 + gn : ws.tab);
    const int32_t pa_in = parent ? pa_raw : gn - 1;
    const float* Sh = Sc + (static_cast<size_t>(bq) * Hv + h) * D * D;
    f4 sv[RT][KS];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int k = 0; k < KS; ++k)
            sv[t][k] = __builtin_nontemporal_load(
                reinterpret_cast<const f4*>(Sh + static_cast<size_t>(rb + 16 * t + c) * D + 16 * k + 4 * q));
    float vv[RT][8];   // slot e: node 4 q + e (e < 4), 16 + 4 q + e - 4 (e >= 4)
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int node = min(e < 4 ? 4 * q + e : 12 + 4 * q + e, n - 1);
            vv[t][e] = ws.v[(static_cast<size_t>(m0 + node) * Hv + h) * D + rb + 16 * t + c];
        }

#pragma unroll
    for (int e = 0; e < QK4; ++e) {
        const int idx = tid + 256 * e, node = idx / (D / 2), f = idx % (D / 2);
        ut_bf4 hi, lo;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            ut_split_at(node < n ? qk[e][j] : 0.0f, hi, lo, j);
        if (f < D / 4) {
            *reinterpret_cast<ut_bf4*>(&sm.qh[node][4 * f]) = hi;
            *reinterpret_cast<ut_bf4*>(&sm.ql[node][4 * f]) = lo;
        } else {
            const int col = 4 * (f - D / 4);
            *reinterpret_cast<ut_bf4*>(&sm.kh[node][col]) = hi;
            *reinterpret_cast<ut_bf4*>(&sm.kl[node][col]) = lo;
        }
    }
    // rho and gamma, while the q/k loads are in flight: lane i of wave 0
    // clears row i of rho and walks up from node i (the gates and parents it
    // reads were written by lanes of the same wave, whose LDS accesses are
    // processed in order).  A block's path is i, i - 1, ..., 0, so its gate
    // loads do not wait on one another.
    if (wave == 0 && lane < NT) {
        sm.al[lane] = lane < n ? al_in : 1.0f;
        sm.be[lane] = lane < n ? be_in : 0.0f;
        sm.par[lane] = lane < n ? pa_in : -1;
#pragma unroll
        for (int l = 0; l < NT; l += 4)
            *reinterpret_cast<f4*>(&sm.rho[lane][l]) = f4{0.0f, 0.0f, 0.0f, 0.0f};
        float prod = 1.0f;
        if (parent == nullptr) {
            if (lane >= n)
                sm.rho[lane][lane] = 1.0f;
            for (int l = lane < n ? lane : -1; l >= 0; --l) {
                sm.rho[lane][l] = prod;
                prod *= sm.al[l];
            }
        } else {
            int cur = lane;
            for (int st = 0; st < NT && cur >= 0 && cur < NT; ++st) {
                sm.rho[lane][cur] = prod;
                prod *= sm.al[cur];
                cur = sm.par[cur];
            }
        }
        sm.gam[lane] = prod;
    }
    __syncthreads();

    // Every wave takes one 16x16 tile (I, J) of K K^T and of Q K^T, and forms
    // A and M on it from the gates on the ancestor paths (rho is 0 off them).
    // Tile (0, 1) lies above the diagonal, where neither has an entry.
    {
        const int I = wave >> 1, J = wave & 1;
        f4 gk0 = {0.0f, 0.0f, 0.0f, 0.0f}, gk1 = gk0, gq0 = gk0, gq1 = gk0;
        if (!(I == 0 && J == 1)) {
#pragma unroll
            for (int m = 0; m < KS / 2; ++m) {
                const int c0 = 32 * m + 4 * q, c1 = c0 + 16;
                const bf8 akh = ut_cat(&sm.kh[16 * I + c][c0], &sm.kh[16 * I + c][c1]);
                const bf8 akl = ut_cat(&sm.kl[16 * I + c][c0], &sm.kl[16 * I + c][c1]);
                const bf8 aqh = ut_cat(&sm.qh[16 * I + c][c0], &sm.qh[16 * I + c][c1]);
                const bf8 aql = ut_cat(&sm.ql[16 * I + c][c0], &sm.ql[16 * I + c][c1]);
                const bf8 bkh = ut_cat(&sm.kh[16 * J + c][c0], &sm.kh[16 * J + c][c1]);
                const bf8 bkl = ut_cat(&sm.kl[16 * J + c][c0], &sm.kl[16 * J + c][c1]);
                gk0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(akh, bkh, gk0, 0, 0, 0);
                gq0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aqh, bkh, gq0, 0, 0, 0);
                gk1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(akh, bkl, gk1, 0, 0, 0);
                gq1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aqh, bkl, gq1, 0, 0, 0);
                gk1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(akl, bkh, gk1, 0, 0, 0);
                gq1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aql, bkh, gq1, 0, 0, 0);
            }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = 16 * I + 4 * q + v, l = 16 * J + c;
            const float r = sm.rho[i][l];
            sm.ga[i][l] = l == i ? 0.0f : sm.be[i] * r * (gk0[v] + gk1[v]);
            sm.gm[i][l] = r * (gq0[v] + gq1[v]);
        }
    }
    __syncthreads();

    // (I + A)^-1: the two diagonal 16x16 blocks by substitution (wave 0, lane =
    // (block, column)); the block above the diagonal is 0.
    if (wave == 0 && lane < NT) {
        const int b0 = 16 * (lane >> 4), j = lane & 15;
        float X[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float arow[16];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const f4 a4 = *reinterpret_cast<const f4*>(&sm.ga[b0 + i][b0 + 4 * p]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    arow[4 * p + e] = a4[e];
            }
            float s = i == j ? 1.0f : 0.0f;
#pragma unroll
            for (int k = 0; k < i; ++k)
                s = __builtin_fmaf(-arow[k], X[k], s);
            X[i] = s;
            sm.t[b0 + i][b0 + j] = s;
        }
    } else if (wave == 1) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
            sm.t[4 * q + v][16 + c] = 0.0f;
    }
    __syncthreads();
    // the block below it: T_10 = -T_11 (A_10 T_00)
    if (wave == 0) {
        f4 z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
            z = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.ga[16 + c][4 * q + s], sm.t[4 * q + s][c], z, 0, 0, 0);
        f4 tt = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
            tt = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.t[16 + c][16 + 4 * q + s], z[s], tt, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v)
            sm.t[16 + 4 * q + v][c] = -tt[v];
    }
    __syncthreads();

    // R = M (I + A)^-1 diag(beta) and R diag(gamma), one 16x16 tile per wave.
    {
        const int I = wave >> 1, J = wave & 1;
        f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if (!(I == 0 && J == 1)) {
#pragma unroll
            for (int K = 0; K < 2; ++K)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.gm[16 * I + c][16 * K + 4 * q + s],
                                                               sm.t[16 * K + 4 * q + s][16 * J + c], acc, 0, 0, 0);
        }
        const float bc = sm.be[16 * J + c], gc = sm.gam[16 * J + c];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float rv = acc[v] * bc;
            sm.r[16 * I + 4 * q + v][16 * J + c] = rv;
            sm.rg[16 * I + 4 * q + v][16 * J + c] = rv * gc;
        }
    }
    __syncthreads();

    // e = gamma q - (R diag(gamma)) K, written over q; and the accumulators of
    // the last product start at R V.  Both on split bf16 MFMA with the 32
    // nodes as k: slot e of lane (q, c) is node 4 q + e, or 16 + 4 q + e - 4.
    auto row_split = [&](const float (*M)[UtWsSmem<D>::PS], int row, bf8& hi, bf8& lo) {
        const f4 x0 = *reinterpret_cast<const f4*>(&M[row][4 * q]);
        const f4 x1 = *reinterpret_cast<const f4*>(&M[row][16 + 4 * q]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ut_split_at(x0[e], hi, lo, e);
            ut_split_at(x1[e], hi, lo, 4 + e);
        }
    };
#pragma unroll
    for (int e = 0; e < ET; ++e) {
        const int tau = wave * ET + e, U = tau & 1, Ct = tau >> 1, col = 16 * Ct + c;
        bf8 ah, al;
        row_split(sm.rg, 16 * U + c, ah, al);
        bf8 bh, bl;   // k of the slot nodes, one column: 2-byte reads down the rows
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int l = e < 4 ? 4 * q + e : 12 + 4 * q + e;
            bh[e] = sm.kh[l][col];
            bl[e] = sm.kl[l][col];
        }
        const f4 z = ut_mma3(ah, al, bh, bl, f4{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = 16 * U + 4 * q + v;
            const float qv = static_cast<float>(sm.qh[i][col]) + static_cast<float>(sm.ql[i][col]);
            ut_split(sm.gam[i] * qv - z[v], sm.qh[i][col], sm.ql[i][col]);
        }
    }
    f4 acc[RT][NTW];
#pragma unroll
    for (int u = 0; u < NTW; ++u) {
        bf8 ah, al;
        row_split(sm.r, 16 * (u0 + u) + c, ah, al);
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            bf8 vh, vl;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                ut_split_at(vv[t][e] * ((e < 4 ? 4 * q + e : 12 + 4 * q + e) < n ? 1.0f : 0.0f), vh, vl, e);
            acc[t][u] = ut_mma3(ah, al, vh, vl, f4{0.0f, 0.0f, 0.0f, 0.0f});
        }
    }
    __syncthreads();

    // o = s (E S_c^T + R V) over this wave's rows, E and the checkpoint rows
    // split alike.  Lane (q, c) holds, for k-step m, the columns 32 m + 4 q +
    // 0..3 and 32 m + 16 + 4 q + 0..3 of its row, in both operands.
#pragma unroll
    for (int m = 0; m < KS / 2; ++m) {
        bf8 shi[RT], slo[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                ut_split_at(sv[t][2 * m + e / 4][e % 4], shi[t], slo[t], e);
#pragma unroll
        for (int u = 0; u < NTW; ++u) {
            const int row = 16 * (u0 + u) + c, c0 = 32 * m + 4 * q;
            const bf8 ah = ut_cat(&sm.qh[row][c0], &sm.qh[row][c0 + 16]);
            const bf8 al = ut_cat(&sm.ql[row][c0], &sm.ql[row][c0 + 16]);
#pragma unroll
            for (int t = 0; t < RT; ++t)
                acc[t][u] = ut_mma3(ah, al, shi[t], slo[t], acc[t][u]);
        }
    }
    if (ws.tab[static_cast<size_t>(bq) * (2 * n + 1) + 2 * n] == 0)
        return;   // malformed tree (reported by the prep): nothing is written
#pragma unroll
    for (int u = 0; u < NTW; ++u)
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int node = 16 * (u0 + u) + 4 * q + v;
                if (node < n)
                    o[(static_cast<size_t>(m0 + node) * Hv + h) * D + rb + 16 * t + c] = Scale<D>::value * acc[t][u][v];
            }
}

// The UT-form verify of a tree, or of a block when parent is null.  With no
// workspace, the one launch; with one, the workspace is filled for a prepared
// commit to read: at small batches by prep workgroups in the same launch as
// the one-launch verify, otherwise by the prep launch, after which the UT
// kernel reads its operands from it.  Measured on the 27B-class layer, the
// one-launch form against prep + workspace UT kernel: 16.0 us against 15.3 at
// one tree, 23.7 against 31.0 at 8, 104 against 120 at 64 (before the
// dot-product conv).
// Up to this batch (bf16 activations) the UT verify with a workspace runs as
// one launch (the one-launch verify beside the prep of the workspace); above
// it, the prep launch and the UT kernel that reads the prepared operands.  Measured on the
// 27B-class layer (32-node trees, graphs of 64 calls), one launch against two:
// 13.3 / 16.4 us at batch 1, 13.9 / 18.2 at 2, 20.5 / 22.1 at 4, 40.3 / 31.2
// at 8 (the prep part's many small workgroups then queue behind the verify's).
constexpr int kUtPrepMaxBatch = 4;
// Up to this many sequences (D = 128) each (sequence, value head) of the UT
// verify is split over two workgroups by rows: at batch 1 and 2 only 48 or 96
// of the 256 CUs would work, and the halves' shorter last step and smaller
// checkpoint share outweigh building the small matrices twice.  Measured on the
// 27B-class layer (32-node trees, graphs of 32 calls, bit-identical outputs),
// split against whole: one launch 10.98 / 12.68 us at batch 1, 11.17 / 12.69
// at 2, 15.01 / 13.36 at 4, 19.80 / 19.17 at 8, 112.1 / 93.0 at 64.
constexpr int kUtSplitMaxBatch = 2;

hipError_t launch_tree_verify_ut(const Geo& g, const float* S, const void* tail, const void* w, int n,
                                 const int32_t* parent, const void* x, const float* a, const float* b, float* o,
                                 int32_t* status, void* ws, hipStream_t s) {
    const bool split = g.D == 128 && g.B <= kUtSplitMaxBatch;
    if (ws == nullptr)
        return dispatch(g, [&](auto dtag, auto atag) {
            constexpr int D = decltype(dtag)::value;
            using Act = decltype(atag);
            if (D == 128 && split)
                hipLaunchKernelGGL((tree_ut_kernel<D, Act, D == 128 ? 2 : 1>), dim3(static_cast<unsigned>(2 * g.B * g.Hv)),
                                   dim3(256), 0, s, S, static_cast<const Act*>(tail), static_cast<const Act*>(w), n,
                                   parent, static_cast<const Act*>(x), a, b, o, status, g.Hk, g.Hv, g.C);
            else
                hipLaunchKernelGGL((tree_ut_kernel<D, Act, 1>), dim3(static_cast<unsigned>(g.B * g.Hv)), dim3(256), 0,
                                   s, S, static_cast<const Act*>(tail), static_cast<const Act*>(w), n, parent,
                                   static_cast<const Act*>(x), a, b, o, status, g.Hk, g.Hv, g.C);
        });
    const TreeWs W = tree_ws_carve(ws, g.B, n, g.Hk, g.Hv, g.D);
    // bf16 activations only: with fp32 ones the verify's staging alone takes
    // half a CU's LDS, and the prep's share would leave one workgroup per CU.
    if (g.B <= kUtPrepMaxBatch && g.bf16)
        return dispatch(g, [&](auto dtag, auto atag) {
            constexpr int D = decltype(dtag)::value;
            using Act = decltype(atag);
            if constexpr (sizeof(Act) == 2) {
                const int prep_blocks = g.B + g.B * g.Hk * n;
                if (D == 128 && split) {
                    const int ut_blocks = 2 * g.B * g.Hv;
                    hipLaunchKernelGGL((tree_ut_prep_kernel<D, Act, D == 128 ? 2 : 1>),
                                       dim3(static_cast<unsigned>(ut_blocks + prep_blocks)), dim3(256), 0, s, S,
                                       static_cast<const Act*>(tail), static_cast<const Act*>(w), n, parent,
                                       static_cast<const Act*>(x), a, b, o, status, W, g.B, g.Hk, g.Hv, g.C,
                                       ut_blocks);
                } else {
                    const int ut_blocks = g.B * g.Hv;
                    hipLaunchKernelGGL((tree_ut_prep_kernel<D, Act, 1>),
                                       dim3(static_cast<unsigned>(ut_blocks + prep_blocks)), dim3(256), 0, s, S,
                                       static_cast<const Act*>(tail), static_cast<const Act*>(w), n, parent,
                                       static_cast<const Act*>(x), a, b, o, status, W, g.B, g.Hk, g.Hv, g.C,
                                       ut_blocks);
                }
            }
        });
    hipError_t e = dispatch(g, [&](auto dtag, auto atag) {
        constexpr int D = decltype(dtag)::value;
        using Act = decltype(atag);
        launch_prep<D, Act>(g, n, tail, w, parent, x, a, b, W, status, s);
    });
    if (e != hipSuccess)
        return e;
    return dispatch(g, [&](auto dtag, auto) {
        constexpr int D = decltype(dtag)::value;
        hipLaunchKernelGGL((tree_ut_ws_kernel<D>), dim3(static_cast<unsigned>(g.B * g.Hv)), dim3(256), 0, s, S, n,
                           parent, W, o, g.Hk, g.Hv);
    });
}

// ------------------------------------------------------------ blocks

// Kernels that rewrite the conv tail themselves give each of a sequence's
// B*Hv*bph workgroups ceil(C / (Hv*bph)) channels, one per thread.  With
// C = 2*Hk*D + Hv*D <= 3*Hv*D that is at most 3*D/bph (96 for both supported
// head widths at their fewest row blocks per head); the launchers refuse a
// geometry where it would exceed 256.
static bool tail_share_fits(const Geo& g, int bph) {
    return (g.C + g.Hv * bph - 1) / (g.Hv * bph) <= 256;
}
static int row_blocks_per_head(const Geo& g) {   // one pass of 4 row groups per workgroup
    return g.D == 128 ? 128 / (4 * Row<128>::RPW) : 32 / (4 * Row<32>::RPW);
}

// From this many (sequence, value head) pairs on, a commit (of a path or of
// a block) gives each wave two row groups.  Measured on the 27B-class layer
// (graphs of 64 calls; prepared / replaying), paths in 32-node trees:
// 82.1 / 105.4 us against 92.5 / 138.3 at 64 sequences, 13.1 / 22.8 against
// 16.4 / 29.4 at 8, 9.8 / 16.7 against 10.0 / 19.3 at 4, the same to within
// 2% at 1 and 2; 16-token blocks, 502 tokens accepted over 64 sequences:
// 94.1 / 113.7 against 118.9 / 133.0.
constexpr int64_t kCommitTwoPassMin = 192;
// From this many pairs on, a block commit gives each wave four row groups (a
// workgroup covers 64 rows, two workgroups per head).  16-token blocks on the
// 27B-class layer, 512 tokens accepted over 64 sequences, prepared: 100.6 /
// 99.0 against 101.7 / 102.0 us (two runs); replaying: 127.1 / 126.3 against
// 128.5 / 126.5.  A path commit from the prepared operands keeps two (four:
// 85.4 against 82.4 us for 64 prepared path commits); the replaying path commit
// takes four here too (101.0 / 101.1 against 106.6 / 106.6 us at 64 paths).
constexpr int64_t kBlockCommitFourPassMin = 3072;

// Block commit from the prepared operands of the block's positions (the prep
// launch's workspace): each sequence's state advances by its first len =
// accepted[seq] positions with decode's per-token arithmetic, so the result is
// the bits of one decode step per position.  The work split is the path
// commit's: one workgroup per (sequence, value head, ROWS rows), the state
// rows streamed once; the positions' q|k, v and gates are staged in LDS with
// one 16-byte load per unit, all in flight together.  The kernel also
// rewrites the conv tail (the last four raw inputs of old tail ++ the first
// len positions): nothing in it reads the old tail, so the sequence's
// workgroups share its C channels out, one thread per channel.  A sequence
// whose len is out of range keeps its state and tail and gets status
// GDN_ERR_INDEX.
// MAXL (8, 16 or 32) bounds the block length, and so the LDS a workgroup
// holds: a shorter bound lets more workgroups share a CU.
template <int D, int ROWS, int MAXL>
struct alignas(16) BlockSmem {
    float qk[MAXL][2 * D];   // q^|k^ of each position
    float v[MAXL][ROWS];     // v of the workgroup's rows
    float kq[MAXL], alpha[MAXL], beta[MAXL];
};

template <int D, typename Act, int MAXL, int PASSES>
__global__ __launch_bounds__(256) void block_commit_kernel(float* __restrict__ S, Act* __restrict__ tail, int k,
                                                           const Act* __restrict__ x,
                                                           const int32_t* __restrict__ accepted,
                                                           float* __restrict__ o, int32_t* __restrict__ status,
                                                           int Hk, int Hv, int C, int blocks_per_head, TreeWs ws) {
    using R = Row<D>;
    constexpr int NV = R::NV, LPR = R::LPR, RPW = R::RPW;
    constexpr int ROWS_PASS = 4 * RPW;
    constexpr int ROWS = ROWS_PASS * PASSES;   // PASSES row groups per wave, as in commit_state_kernel
    static_assert(ROWS <= D, "a workgroup's rows lie in one head");
    __shared__ BlockSmem<D, ROWS, MAXL> sm;
    asm volatile("" : "+s"(blocks_per_head) : "s"(S), "s"(tail), "s"(k), "s"(x), "s"(accepted), "s"(o), "s"(status),
                 "s"(Hk), "s"(Hv), "s"(C));
    const int wid = xcd_packed_id(blockIdx.x, gridDim.x);
    const int blk = wid % blocks_per_head;
    const int h = (wid / blocks_per_head) % Hv;
    const int bq = wid / (blocks_per_head * Hv);
    const int grp = h / (Hv / Hk);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r = lane % LPR;
    const int row0 = blk * ROWS;
    int lrow[PASSES];   // the lane's row in each pass, within the workgroup's rows
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
        lrow[p] = p * ROWS_PASS + wave * RPW + lane / LPR;
    float* Sh = S + (static_cast<size_t>(bq) * Hv + h) * D * D;
    float4 s[PASSES][NV];
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
#pragma unroll
        for (int j = 0; j < NV; ++j)
            s[p][j] = load_stream(Sh + (row0 + lrow[p]) * D + R::key(j, r));
    const int len = accepted[bq];
    const bool valid = len >= 0 && len <= k;
    if (status && wid % (blocks_per_head * Hv) == 0 && threadIdx.x == 0)
        status[bq] = valid ? 0 : 10;   // GDN_ERR_INDEX
    if (!valid || len == 0)
        return;

    // This thread's tail channel (the sequence's workgroups share the C
    // channels out: at most 192 per workgroup for the supported head widths)
    // and its last four inputs, loaded with the operands.
    const int per = (C + blocks_per_head * Hv - 1) / (blocks_per_head * Hv);
    const int tc = (wid % (blocks_per_head * Hv)) * per + static_cast<int>(threadIdx.x);
    const bool tail_writer = static_cast<int>(threadIdx.x) < per && tc < C;
    const int tcc = tail_writer ? tc : 0;
    using Q = Quad<Act>;
    Act* tp = tail + (static_cast<size_t>(bq) * C + tcc) * 4;
    const typename Q::raw told = Q::load(tp);
    Act xin[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int j = len - 4 + e;
        xin[e] = x[(static_cast<size_t>(bq) * k + (j < 0 ? 0 : j)) * C + tcc];
    }

    // The positions' operands: q|k of the q/k head, v of this workgroup's
    // rows, (alpha, beta, k.q) of the value head; one 16-byte unit per load.
    constexpr int U = D / 2 + ROWS / 4 + 1;             // units per position
    constexpr int NL = (MAXL * U + 255) / 256;          // units per thread
    float4 un[NL];
#pragma unroll
    for (int e = 0; e < NL; ++e) {
        const int idx = min(static_cast<int>(threadIdx.x) + 256 * e, len * U - 1), i = idx / U, f = idx % U;
        const size_t m = static_cast<size_t>(bq) * k + i;
        const float* src = f < D / 2 ? ws.qk + (m * Hk + grp) * 2 * D + 4 * f
                           : f < D / 2 + ROWS / 4 ? ws.v + (m * Hv + h) * D + row0 + 4 * (f - D / 2)
                                                  : ws.abk + (m * Hv + h) * 4;
        un[e] = *reinterpret_cast<const float4*>(src);
    }
#pragma unroll
    for (int e = 0; e < NL; ++e) {
        const int idx = threadIdx.x + 256 * e, i = idx / U, f = idx % U;
        if (idx < len * U) {
            if (f < D / 2) {
                *reinterpret_cast<float4*>(&sm.qk[i][4 * f]) = un[e];
            } else if (f < D / 2 + ROWS / 4) {
                *reinterpret_cast<float4*>(&sm.v[i][4 * (f - D / 2)]) = un[e];
            } else {
                sm.alpha[i] = un[e].x;
                sm.beta[i] = un[e].y;
                sm.kq[i] = un[e].z;
            }
        }
    }
    __syncthreads();
    if (tail_writer) {
        typename Q::raw t = told;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (len - 4 + e >= 0)
                t = Q::push(t, xin[e]);
        Q::store(tp, t);
    }

    float* ob = o ? o + static_cast<size_t>(bq) * k * Hv * D : nullptr;
    TokOps<D> cur, nxt;   // v of pass 0 in .v, of the others in cv / nv
    float cv[PASSES], nv[PASSES];
    auto load_tok = [&](TokOps<D>& t, float (&vp)[PASSES], int i) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            t.k[j] = *reinterpret_cast<const float4*>(&sm.qk[i][D + R::key(j, r)]);
            t.q[j] = *reinterpret_cast<const float4*>(&sm.qk[i][R::key(j, r)]);
        }
        t.v = sm.v[i][lrow[0]];
#pragma unroll
        for (int p = 1; p < PASSES; ++p)
            vp[p] = sm.v[i][lrow[p]];
        t.alpha = sm.alpha[i];
        t.beta = sm.beta[i];
        t.kq = sm.kq[i];
    };
    load_tok(cur, cv, 0);
    for (int i = 0; i < len; ++i) {
        load_tok(nxt, nv, i + 1 < len ? i + 1 : i);
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const float out =
                row_update<D>(s[p], cur.k, cur.q, cur.alpha, cur.beta, p == 0 ? cur.v : cv[p], cur.kq);
            if (ob && r == 0)
                ob[(static_cast<size_t>(i) * Hv + h) * D + row0 + lrow[p]] = out;
        }
        cur = nxt;
#pragma unroll
        for (int p = 1; p < PASSES; ++p)
            cv[p] = nv[p];
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
#pragma unroll
        for (int j = 0; j < NV; ++j)
            store_stream(Sh + (row0 + lrow[p]) * D + R::key(j, r), s[p][j]);
}

// prepared: the workspace already holds the block's operands (from the
// verify of the same block), so the prep launch is skipped.
hipError_t launch_block(const Geo& g, bool commit, float* S, void* tail, const void* w, int k, const void* x,
                        const float* a, const float* b, const int32_t* accepted, float* o, int32_t* status, void* ws,
                        bool prepared, hipStream_t s) {
    const bool two = commit && g.D == 128 && static_cast<int64_t>(g.B) * g.Hv >= kCommitTwoPassMin;
    const bool four = two && static_cast<int64_t>(g.B) * g.Hv >= kBlockCommitFourPassMin;
    const int cbph = row_blocks_per_head(g) / (four ? 4 : two ? 2 : 1);   // row blocks per head of the commit
    if (commit && !tail_share_fits(g, cbph))
        return hipErrorInvalidValue;
    const TreeWs W = tree_ws_carve(ws, g.B, k, g.Hk, g.Hv, g.D);
    hipError_t e = prepared ? hipSuccess : dispatch(g, [&](auto dtag, auto atag) {
        constexpr int D = decltype(dtag)::value;
        using Act = decltype(atag);
        launch_prep<D, Act>(g, k, tail, w, nullptr, x, a, b, W, nullptr, s);
    });
    if (e != hipSuccess)
        return e;
    return dispatch(g, [&](auto dtag, auto atag) {
        constexpr int D = decltype(dtag)::value;
        using Act = decltype(atag);
        const int bph = D / (4 * Row<D>::RPW);
        const unsigned grid = static_cast<unsigned>(g.B * g.Hv * bph);
        auto commit_go = [&](auto ptag) {
            constexpr int PASSES = decltype(ptag)::value;
            const dim3 cgrid(static_cast<unsigned>(g.B * g.Hv * cbph));
            if (k <= 8)
                hipLaunchKernelGGL((block_commit_kernel<D, Act, 8, PASSES>), cgrid, dim3(256), 0, s, S,
                                   static_cast<Act*>(tail), k, static_cast<const Act*>(x), accepted, o, status, g.Hk,
                                   g.Hv, g.C, cbph, W);
            else if (k <= 16)
                hipLaunchKernelGGL((block_commit_kernel<D, Act, 16, PASSES>), cgrid, dim3(256), 0, s, S,
                                   static_cast<Act*>(tail), k, static_cast<const Act*>(x), accepted, o, status, g.Hk,
                                   g.Hv, g.C, cbph, W);
            else
                hipLaunchKernelGGL((block_commit_kernel<D, Act, kMaxNodes, PASSES>), cgrid, dim3(256), 0, s, S,
                                   static_cast<Act*>(tail), k, static_cast<const Act*>(x), accepted, o, status, g.Hk,
                                   g.Hv, g.C, cbph, W);
        };
        if (commit) {
            if constexpr (D == 128) {
                if (four) {
                    commit_go(std::integral_constant<int, 4>{});
                    return;
                }
                if (two) {
                    commit_go(std::integral_constant<int, 2>{});
                    return;
                }
            }
            commit_go(std::integral_constant<int, 1>{});
        } else if (grid > 2u * 256u)
            hipLaunchKernelGGL((tree_verify_kernel<D, WalkWide, WalkKind::Chain>), dim3(grid), dim3(256), 0, s, S, k,
                               W, o, g.Hk, g.Hv, bph);
        else
            hipLaunchKernelGGL((tree_verify_kernel<D, WalkDeep, WalkKind::Chain>), dim3(grid), dim3(256), 0, s, S, k,
                               W, o, g.Hk, g.Hv, bph);
    });
}

// ------------------------------------------------------------ commit

// PREPARED: the operands come from the verify's workspace, so no workgroup
// reads the tail, and the kernel also rewrites it (tail_out, the same buffer):
// each channel by one thread, after the path is validated.  Otherwise the
// conv reads the tail here and commit_tail_kernel rewrites it afterwards.
// PASSES: row groups per wave (a workgroup covers 4 * RPW * PASSES rows).  Two
// halve the per-row share of the path's operand loads and the validation, and
// give each token's replay two independent row updates.
template <int D, typename Act, bool PREPARED, int PASSES>
__global__ __launch_bounds__(256) void commit_state_kernel(float* __restrict__ S, const Act* __restrict__ tail,
                                                           Act* __restrict__ tail_out, const Act* __restrict__ w,
                                                           int n,
                                                           const int32_t* __restrict__ parent,
                                                           const Act* __restrict__ x, const float* __restrict__ a,
                                                           const float* __restrict__ b, int L,
                                                           const int32_t* __restrict__ path, float* __restrict__ o,
                                                           int32_t* __restrict__ status, int Hk, int Hv, int C,
                                                           int blocks_per_head, TreeWs ws) {
    using R = Row<D>;
    constexpr int NV = R::NV, LPR = R::LPR, RPW = R::RPW;
    constexpr int ROWS_PASS = 4 * RPW;
    constexpr int ROWS = ROWS_PASS * PASSES;
    static_assert(ROWS <= D, "a workgroup's rows lie in one head");
    __shared__ NodeSmem<D, ROWS, kMaxDepth, Act> sm;

    // The index arithmetic is made to depend on every argument, so all the
    // argument loads issue together (one kernel-argument round trip).
    asm volatile("" : "+s"(blocks_per_head) : "s"(S), "s"(tail), "s"(tail_out), "s"(w), "s"(n), "s"(parent), "s"(x),
                 "s"(a), "s"(b), "s"(L), "s"(path), "s"(o), "s"(status), "s"(Hk), "s"(Hv), "s"(C));
    // Workgroups of one (sequence, q/k head) share their token inputs; they
    // are kept on one XCD.
    const int wid = xcd_packed_id(blockIdx.x, gridDim.x);
    const int blk = wid % blocks_per_head;
    const int h = (wid / blocks_per_head) % Hv;
    const int bq = wid / (blocks_per_head * Hv);
    const int grp = h / (Hv / Hk);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r = lane % LPR;
    const int row0 = blk * ROWS;
    int lrow[PASSES];   // the lane's row in each pass, within the workgroup's rows
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
        lrow[p] = p * ROWS_PASS + wave * RPW + lane / LPR;
    parent += static_cast<size_t>(bq) * n;
    path += static_cast<size_t>(bq) * L;
    x += static_cast<size_t>(bq) * n * C;
    a += static_cast<size_t>(bq) * n * Hv;
    b += static_cast<size_t>(bq) * n * Hv;
    tail += static_cast<size_t>(bq) * C * 4;
    tail_out += PREPARED ? static_cast<size_t>(bq) * C * 4 : 0;

    float* Sh = S + (static_cast<size_t>(bq) * Hv + h) * D * D;
    float4 s[PASSES][NV];
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
#pragma unroll
        for (int j = 0; j < NV; ++j)
            s[p][j] = load_stream(Sh + (row0 + lrow[p]) * D + R::key(j, r));

    // Token i of the commit is path position i; its ancestors are the
    // positions before it.  The row's length is the index of its first -1.
    // Node ids are clamped into the tree so that every load below stays in
    // bounds whatever the path holds; a malformed path is rejected before
    // anything is written.
    if (wave == 0) {
        const int len = path_len_wave(L, path);
        if (lane < kMaxDepth) {
            int nd = path[lane < L ? lane : L - 1];
            nd = nd < 0 ? 0 : nd >= n ? n - 1 : nd;
            sm.node[lane] = nd;
            sm.depth[lane] = lane + 1;
#pragma unroll
            for (int k = 1; k <= 3; ++k)
                sm.anc[lane][k - 1] = lane - k;
        }
        if (lane == 0)
            sm.len = len;
    }
    __syncthreads();
    const int len = sm.len;
    const int cnt = len > 0 ? len : 1;   // tokens loaded and convolved (in bounds for the empty path)
    auto validate = [&]() {   // wave 0; overlaps the loads just issued
        bool ok = tree_tables_wave(n, parent, nullptr, nullptr);
        ok = ok && path_check_wave(n, parent, L, path);
        if (lane == 0) {
            sm.ok = ok ? 1 : 0;
            if (status && wid % (blocks_per_head * Hv) == 0)
                status[bq] = ok ? 0 : 5;
        }
    };
    if constexpr (!PREPARED) {
        FillRegs<D, ROWS, kMaxDepth, Act> fr;
        fill_issue<D, ROWS, kMaxDepth, Act>(fr, sm, cnt, x, tail, w, a, b, Hk, Hv, C, grp, h, row0);
        if (wave == 0)
            validate();
        fill_finish<D, ROWS, kMaxDepth, Act>(fr, sm, cnt);
    } else {
        // The path's operands as the verify's prep launch left them in the
        // workspace (normalised q|k, v of this workgroup's rows, alpha, beta,
        // k.q): every token's loads in flight at once, then into LDS.
        constexpr int U = D / 2 + ROWS / 4 + 1;              // 16-byte units per token
        constexpr int NL = (kMaxDepth * U + 255) / 256;      // units per thread
        // This thread's tail channel (the sequence's workgroups share them out):
        // its old entries and the path tokens' inputs, loaded with the operands.
        const int per = (C + blocks_per_head * Hv - 1) / (blocks_per_head * Hv);
        const int tc = (wid % (blocks_per_head * Hv)) * per + static_cast<int>(threadIdx.x);
        const bool tail_writer = static_cast<int>(threadIdx.x) < per && tc < C;
        const int tcc = tail_writer ? tc : 0;
        using Q = Quad<Act>;
        const typename Q::raw told = Q::load(tail_out + static_cast<size_t>(tcc) * 4);
        Act xin[kMaxDepth];
#pragma unroll
        for (int j = 0; j < kMaxDepth; ++j)
            xin[j] = x[static_cast<size_t>(sm.node[j]) * C + tcc];
        float4 un[NL];
#pragma unroll
        for (int e = 0; e < NL; ++e) {
            const int idx = min(static_cast<int>(threadIdx.x) + 256 * e, cnt * U - 1), i = idx / U, f = idx % U;
            const size_t m = static_cast<size_t>(bq) * n + sm.node[i];
            const float* src = f < D / 2 ? ws.qk + (m * Hk + grp) * 2 * D + 4 * f
                               : f < D / 2 + ROWS / 4 ? ws.v + (m * Hv + h) * D + row0 + 4 * (f - D / 2)
                                                      : ws.abk + (m * Hv + h) * 4;
            un[e] = *reinterpret_cast<const float4*>(src);
        }
        if (wave == 0)
            validate();
#pragma unroll
        for (int e = 0; e < NL; ++e) {
            const int idx = threadIdx.x + 256 * e, i = idx / U, f = idx % U;
            if (idx < cnt * U) {
                if (f < D / 2) {
                    *reinterpret_cast<float4*>(&sm.qk[i][4 * f]) = un[e];
                } else if (f < D / 2 + ROWS / 4) {
                    *reinterpret_cast<float4*>(&sm.v[i][4 * (f - D / 2)]) = un[e];
                } else {
                    sm.alpha[i] = un[e].x;
                    sm.beta[i] = un[e].y;
                    sm.kq[i] = un[e].z;
                }
            }
        }
        __syncthreads();
        if (sm.ok && len > 0 && tail_writer) {
            typename Q::raw t = told;
#pragma unroll
            for (int j = 0; j < kMaxDepth; ++j)
                if (j < len)
                    t = Q::push(t, xin[j]);
            Q::store(tail_out + static_cast<size_t>(tc) * 4, t);
        }
    }
    if (!sm.ok || len == 0)
        return;

    float* ob = o ? o + static_cast<size_t>(bq) * L * Hv * D : nullptr;
    TokOps<D> cur, nxt;   // v of pass 0 in .v, of the others in cv / nv
    float cv[PASSES], nv[PASSES];
    tok_load(cur, sm, 0, r, lrow[0]);
#pragma unroll
    for (int p = 1; p < PASSES; ++p)
        cv[p] = sm.v[0][lrow[p]];
    for (int i = 0; i < len; ++i) {
        const int i1 = i + 1 < len ? i + 1 : i;
        tok_load(nxt, sm, i1, r, lrow[0]);
#pragma unroll
        for (int p = 1; p < PASSES; ++p)
            nv[p] = sm.v[i1][lrow[p]];
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const float out =
                row_update<D>(s[p], cur.k, cur.q, cur.alpha, cur.beta, p == 0 ? cur.v : cv[p], cur.kq);
            if (ob && r == 0)
                ob[(static_cast<size_t>(i) * Hv + h) * D + row0 + lrow[p]] = out;
        }
        cur = nxt;
#pragma unroll
        for (int p = 1; p < PASSES; ++p)
            cv[p] = nv[p];
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
#pragma unroll
        for (int j = 0; j < NV; ++j)
            store_stream(Sh + (row0 + lrow[p]) * D + R::key(j, r), s[p][j]);
}

// The tail after a commit holds the last four raw inputs of (old tail ++ path).
// Path node ids are clamped into the tree so the loads can be issued before
// the path is validated; nothing is written unless it is valid.
template <typename Act>
__global__ __launch_bounds__(256) void commit_tail_kernel(Act* __restrict__ tail, int n,
                                                          const int32_t* __restrict__ parent,
                                                          const Act* __restrict__ x, int L,
                                                          const int32_t* __restrict__ path, int C) {
    __shared__ int32_t ok_s, len_s;
    const int bq = blockIdx.y;   // sequence
    parent += static_cast<size_t>(bq) * n;
    path += static_cast<size_t>(bq) * L;
    x += static_cast<size_t>(bq) * n * C;
    tail += static_cast<size_t>(bq) * C * 4;
    const int c0 = blockIdx.x * blockDim.x + threadIdx.x;
    const int c = c0 < C ? c0 : C - 1;
    using Q = Quad<Act>;
    typename Q::raw t = Q::load(tail + static_cast<size_t>(c) * 4);
    Act xin[kMaxDepth];
#pragma unroll
    for (int j = 0; j < kMaxDepth; ++j) {
        int nd = path[j < L ? j : L - 1];
        nd = nd < 0 ? 0 : nd >= n ? n - 1 : nd;
        xin[j] = x[static_cast<size_t>(nd) * C + c];
    }
    if (threadIdx.x < kWave) {
        bool ok = tree_tables_wave(n, parent, nullptr, nullptr);
        ok = ok && path_check_wave(n, parent, L, path);
        const int len = path_len_wave(L, path);
        if (threadIdx.x == 0) {
            ok_s = ok ? 1 : 0;
            len_s = len;
        }
    }
    __syncthreads();
    const int len = len_s;
    if (!ok_s || len == 0 || c0 >= C)
        return;
#pragma unroll
    for (int j = 0; j < kMaxDepth; ++j)
        if (j < len)
            t = Q::push(t, xin[j]);
    Q::store(tail + static_cast<size_t>(c) * 4, t);
}

// With a workspace the path's operands come from the preceding verify's prep
// launch instead of being convolved again.
hipError_t launch_commit(const Geo& g, float* S, void* tail, const void* w, int n, const int32_t* parent,
                         const void* x, const float* a, const float* b, int L, const int32_t* path, float* o,
                         int32_t* status, void* ws, hipStream_t s) {
    // Two passes per wave (half as many workgroups) once the batch fills the chip;
    // four in the replaying form at the block commit's threshold, where fewer
    // workgroups also means fewer convolutions of the path's tokens.
    const bool two = g.D == 128 && static_cast<int64_t>(g.B) * g.Hv >= kCommitTwoPassMin;
    const bool four = two && ws == nullptr && static_cast<int64_t>(g.B) * g.Hv >= kBlockCommitFourPassMin;
    const int bph = row_blocks_per_head(g) / (four ? 4 : two ? 2 : 1);
    if (ws != nullptr && !tail_share_fits(g, bph))
        return hipErrorInvalidValue;
    hipError_t e = dispatch(g, [&](auto dtag, auto atag) {
        constexpr int D = decltype(dtag)::value;
        using Act = decltype(atag);
        auto go = [&](auto ptag) {
            constexpr int PASSES = decltype(ptag)::value;
            const dim3 grid(static_cast<unsigned>(g.B * g.Hv * bph));
            if (ws == nullptr)
                hipLaunchKernelGGL((commit_state_kernel<D, Act, false, PASSES>), grid, dim3(256), 0, s, S,
                                   static_cast<const Act*>(tail), nullptr, static_cast<const Act*>(w), n, parent,
                                   static_cast<const Act*>(x), a, b, L, path, o, status, g.Hk, g.Hv, g.C, bph,
                                   TreeWs{});
            else
                hipLaunchKernelGGL((commit_state_kernel<D, Act, true, PASSES>), grid, dim3(256), 0, s, S, nullptr,
                                   static_cast<Act*>(tail), nullptr, n, parent, static_cast<const Act*>(x), nullptr,
                                   nullptr, L, path, o, status, g.Hk, g.Hv, g.C, bph,
                                   tree_ws_carve(ws, g.B, n, g.Hk, g.Hv, g.D));
        };
        if constexpr (D == 128) {
            if (four) {
                go(std::integral_constant<int, 4>{});
                return;
            }
            if (two) {
                go(std::integral_constant<int, 2>{});
                return;
            }
        }
        go(std::integral_constant<int, 1>{});
    });
    if (e != hipSuccess || ws != nullptr)   // the prepared form rewrote the tail itself
        return e;
    const dim3 grid(static_cast<unsigned>((g.C + 255) / 256), static_cast<unsigned>(g.B)), block(256);
    if (g.bf16)
        hipLaunchKernelGGL(commit_tail_kernel<uint16_t>, grid, block, 0, s, static_cast<uint16_t*>(tail), n, parent,
                           static_cast<const uint16_t*>(x), L, path, g.C);
    else
        hipLaunchKernelGGL(commit_tail_kernel<float>, grid, block, 0, s, static_cast<float*>(tail), n, parent,
                           static_cast<const float*>(x), L, path, g.C);
    return hipGetLastError();
}

}  // namespace gdn
