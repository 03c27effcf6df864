// gdn_tree.hpp -- device-side analysis of a draft tree and of an accepted path.
//
// A draft tree arrives as a parent array in device memory (repository
// "Architecture" page, decode-loop diagram: the drafters propose a tree of up
// to 32 nodes after the last committed token).  Node 0 is the root; every
// other node's parent comes earlier.  The kernels need each node's depth and a
// depth-first pre-order, in which a node's ancestors are exactly the nodes on
// the current root-to-node stack.  One wave computes both without a serial
// walk: lane i follows its own ancestor chain (through lane shuffles), packs
// the root-first chain into a 48-bit key, and its pre-order position is the
// number of keys below its own.
#pragma once

#include "gdn_core.hpp"

namespace gdn {

// Checks the tree and fills depth_s[n] and order_s[n] (shared memory; either
// may be null).  Must run on one whole wave; the result is wave-uniform.
__device__ inline bool tree_tables_wave(int n, const int32_t* __restrict__ parent, int32_t* depth_s,
                                        int32_t* order_s) {
    const int lane = threadIdx.x & (kWave - 1);
    const bool live = lane < n;
    const int p = live ? parent[lane] : -1;
    bool bad = live && ((lane == 0) ? (p != -1) : (p < 0 || p >= lane));
    if (__any(bad))
        return false;
    // Chase the chain: c_0 = lane, c_1 = parent, ...; pack (c_i + 1) at 6*i bits.
    int cur = live ? lane : -1;
    int depth = 0;
    uint64_t packed = 0;
#pragma unroll
    for (int step = 0; step <= kMaxDepth; ++step) {
        if (cur >= 0) {
            packed |= static_cast<uint64_t>(cur + 1) << (6 * step);
            ++depth;
        }
        const int up = __shfl(p, cur >= 0 ? cur : 0, kWave);
        cur = (cur >= 0) ? up : -1;
    }
    bad = live && (depth > kMaxDepth || cur >= 0);
    if (__any(bad))
        return false;
    // Root-first key: the root lands in the top slot, shorter chains pad with zeros.
    const uint64_t key = live ? (packed << (6 * (kMaxDepth - depth))) : ~0ull;
    const uint32_t klo = static_cast<uint32_t>(key), khi = static_cast<uint32_t>(key >> 32);
    int rank = 0;
    for (int j = 0; j < n; ++j) {
        const uint64_t kj = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(khi, j))) << 32) |
                            static_cast<uint32_t>(__builtin_amdgcn_readlane(klo, j));
        rank += (kj < key) ? 1 : 0;
    }
    if (live) {
        if (depth_s)
            depth_s[lane] = depth;
        if (order_s)
            order_s[rank] = lane;
    }
    return true;
}

// An accepted-path row of up to L entries holds the path root first, then -1
// in every entry after its end, so sequences of one batch can accept paths of
// different lengths.  Its length is the index of its first -1 (L if none).
// Must run on one whole wave; the result is wave-uniform.
__device__ inline int path_len_wave(int L, const int32_t* __restrict__ path) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint64_t ends = __ballot(lane < L && path[lane < L ? lane : 0] == -1);
    return ends ? __builtin_ctzll(ends) : L;
}

// Checks an accepted-path row: path[0] == 0 and parent[path[j]] == path[j-1]
// up to its end, and only -1 after it (a row of -1 only is the empty path).
// Assumes the tree itself already passed tree_tables_wave.  One whole wave.
__device__ inline bool path_check_wave(int n, const int32_t* __restrict__ parent, int L,
                                       const int32_t* __restrict__ path) {
    const int lane = threadIdx.x & (kWave - 1);
    const int len = path_len_wave(L, path);
    const int pj = (lane < L) ? path[lane] : 0;
    const bool in_range = pj >= 0 && pj < n;
    const int par = (lane < len && in_range) ? parent[pj] : -1;
    const int prev = __shfl(pj, lane > 0 ? lane - 1 : 0, kWave);
    bool bad = false;
    if (lane < len)
        bad = !in_range || ((lane == 0) ? (pj != 0) : (par != prev));
    else if (lane < L)
        bad = pj != -1;
    return !__any(bad);
}

// Workgroup id in an order that keeps consecutive ids on one XCD: the
// dispatcher deals workgroups to the 8 XCDs round robin, so XCD x receives
// blocks x, x + 8, ...; they become one contiguous run of ids.  A bijection
// on [0, nblocks) for any nblocks.
__device__ __forceinline__ int xcd_packed_id(int bid, int nblocks) {
    const int q = nblocks / 8, r = nblocks % 8;
    const int x = bid % 8, k = bid / 8;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + k;
}

// Raw inputs of the conv window that ends at a node of depth d (root = 1):
// the history is tail[0..3] followed by the root-first path; the window is its
// last four entries.  anc[k-1] is the ancestor k steps up (k = 1..3).
template <typename Act>
__device__ __forceinline__ void node_window(const Act* __restrict__ x, const Act* __restrict__ tail, int C, int c,
                                            int node, int d, const int anc[3], float win[4]) {
    // One unconditional load per tap, from a selected address, so all four
    // loads are in flight together.
    win[3] = widen(x[static_cast<size_t>(node) * C + c]);
#pragma unroll
    for (int k = 1; k <= 3; ++k) {
        const Act* src = (k <= d - 1) ? x + static_cast<size_t>(anc[k - 1]) * C + c
                                      : tail + static_cast<size_t>(c) * 4 + (3 + d - k);
        win[3 - k] = widen(*src);
    }
}

}  // namespace gdn
