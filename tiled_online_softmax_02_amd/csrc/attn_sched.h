// attn_sched.h -- the order in which workgroups take their work items, shared by the kernels (device)
// and by the launchers and the CPU tests (host).
//
// The hardware hands consecutive workgroups to the XCDs of the chip in turn (nx of them, each with its
// own L2).  Work that reads the same K and V (one head) should stay on one XCD, and under the causal
// mask the longest tiles should go out first.
#pragma once

#include <hip/hip_runtime.h>

namespace attn {

// Work id of dispatch index g in a grid of G workgroups such that every XCD receives a contiguous
// range of work ids (work that shares K/V then shares an L2).
__host__ __device__ inline int xcd_remap(int g, int G, int nx)
{
    const int per = G / nx, rem = G % nx;
    const int x = g % nx, i = g / nx;
    return x * per + (x < rem ? x : rem) + i;
}

// Work item of workgroup g when the grid holds n_heads * n_tiles workgroups: a head and the position t
// of its tile in issue order (t = 0 goes out first).  When n_heads is a multiple of the XCD count,
// items go out position-major (position 0 of every head, then position 1, ...): dispatch is then
// longest-first over the whole grid when position 0 is the largest tile, and head h always lands on
// XCD h % nx.  Otherwise every XCD takes a contiguous head-major range of items.
__host__ __device__ inline void work_item_of(int g, int G, int n_tiles, int nx, int &head, int &t)
{
    const int n_heads = G / n_tiles;
    if (n_heads % nx == 0) {
        t = g / n_heads;
        head = g - t * n_heads;
    } else {
        const int id = xcd_remap(g, G, nx);
        head = id / n_tiles;
        t = id - head * n_tiles;
    }
}

// Item that workgroup g of a persistent grid of P workgroups takes in round r, when items are in
// longest-first order and round r covers items r P .. r P + P - 1.  In odd rounds the order is reversed
// within each XCD (g = x + nx c takes x + nx (P/nx - 1 - c)), so a workgroup that had one of the
// longest items of a round gets one of the shortest of the next; item j keeps j % nx == g % nx, so a
// head stays on the XCD it started on.  P is a multiple of nx whenever the grid is persistent.
__host__ __device__ inline int persistent_item(int r, int g, int P, int nx)
{
    if ((r & 1) == 0 || P % nx != 0) return r * P + g;
    return r * P + g % nx + nx * (P / nx - 1 - g / nx);
}

// Workgroups of a persistent grid for n_items items over n_heads heads on a device of `cus` compute
// units in nx XCDs, one resident workgroup per compute unit: the largest multiple of nx not above cus,
// or 0 (one workgroup per item) when the items fit in one round or the heads do not spread evenly
// over the XCDs.
__host__ __device__ inline long long persistent_grid(long long n_items, long long n_heads, int cus, int nx)
{
    if (nx < 1 || cus < nx) return 0;
    const long long P = (long long)(cus / nx) * nx;
    return (n_items > P && n_heads % nx == 0) ? P : 0;
}

// Causal forward: pair each workgroup's long and short query block (T-1-p, then p) only while the
// paired grid, n_heads * ceil(T / 2) workgroups of equal work, still fills the `slots` workgroups
// the device holds at once.  Below that a paired grid leaves compute units idle for its whole run,
// and one query block per workgroup, issued longest-first, finishes sooner.
__host__ __device__ inline bool causal_pairs(long long n_heads, int n_qtiles, long long slots)
{
    return n_heads * ((n_qtiles + 1) / 2) >= slots;
}

}  // namespace attn
