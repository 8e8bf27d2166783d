// Weight gradient of one shard's masked lookup: the adjoint of embed.hip.
//
// Method: MiniMind-Tron "5 Vocab Parallelism", 5.2.1 defines the lookup (an owned
// id reads row id - start of the shard, any other id gives a zero row).  The
// lookup is linear in the shard's weight, and its weight gradient scatters the
// output gradient back: every owned token adds dout[i] to row ids[i] - start,
// repeated ids accumulate and off-shard tokens add nothing.
//
// Deterministic, with no floating-point atomics.  Zipf-distributed ids repeat a
// few rows thousands of times, so atomics would both serialise on those rows and
// make the fp32 sums depend on timing.  Instead:
//   1. a stable LSD radix sort of (key, token) with key = id - start for owned ids
//      and key = Vs for the rest (they sort last), 8 bits per pass over
//      bit_width(Vs) bits.  A pass is three kernels: per-tile digit counts, one
//      exclusive scan of the counts in digit-major order, and a stable scatter
//      whose ranks come from wave ballots (tokens keep their order within a key);
//   2. segment_sum_kernel: one wave per block of kSegRows sorted positions x 512 columns.  A
//      row whose tokens all lie in one block is summed in token order and added
//      to dw; the pieces of rows that cross a block edge go to per-block partials;
//   3. segment_fixup_kernel: the block where such a row starts adds its pieces in
//      block order and adds the total to dw.
// Each row of dw is read and written once, by one workgroup per column block.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace vp {

namespace {

constexpr int kRadixBits = 8;
constexpr int kRadix = 1 << kRadixBits;
constexpr int kSortThreads = 256;                      // 4 waves
constexpr int kSortRounds = 4;                         // elements per thread
constexpr int kScanThreads = 1024;
constexpr int kSortTile = kSortThreads * kSortRounds;  // elements per workgroup
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kSortSegs = kSortRounds * kSortWaves;    // (round, wave) groups, in element order

constexpr int kSegRows = 64;        // sorted positions per segment-sum block
constexpr int kSegThreads = 64;     // one wave
constexpr int kSegCols = 8 * kSegThreads;   // columns per block (8 bf16 = 16 bytes per thread)
constexpr int kSegBatch = 16;       // dout rows (and the dw rows they finish) in flight per thread
constexpr int64_t kSegMaxGrid = 1 << 20;   // segment-sum workgroups per launch (grid-stride beyond)

// Sort key of element e: in the first pass it is made from the id, later passes
// read the previous pass's output.
struct KeySource {
    const int64_t *ids;      // first pass only
    const uint32_t *keys;    // later passes
    const uint32_t *vals;    // later passes (token index); the first pass uses e
    int64_t start;
    uint32_t vs;

    __device__ __forceinline__ uint32_t key(int64_t e) const {
        if (keys) return keys[e];
        const int64_t id = ids[e];
        return (id >= start && id - start < (int64_t)vs) ? (uint32_t)(id - start) : vs;
    }
    __device__ __forceinline__ uint32_t val(int64_t e) const { return vals ? vals[e] : (uint32_t)e; }
};

// hist[d * nblk + b] = number of elements of tile b whose digit is d.
__global__ __launch_bounds__(kSortThreads) void radix_count_kernel(KeySource src, int64_t n,
                                                                   int shift, uint32_t *hist,
                                                                   int nblk) {
    __shared__ uint32_t cnt[kRadix];
    const int t = threadIdx.x;
    if (t < kRadix) cnt[t] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kSortTile;
#pragma unroll
    for (int r = 0; r < kSortRounds; ++r) {
        const int64_t e = base + r * kSortThreads + t;
        if (e < n) atomicAdd(&cnt[(src.key(e) >> shift) & (kRadix - 1)], 1u);
    }
    __syncthreads();
    if (t < kRadix) hist[(int64_t)t * nblk + blockIdx.x] = cnt[t];
}

// In-place exclusive scan of `count` values by one workgroup: thread t takes a contiguous
// chunk (16-byte loads, kScanBatch in flight), the chunk sums are scanned across the
// workgroup (within each wave by shuffles, then over the waves' totals in LDS, one
// barrier), and each thread rewrites its chunk.  Chunks of up to kScanBatch x 4 values
// stay in registers between the two; longer ones are read again.  count is a multiple
// of 4 (kRadix x tiles) and hist is 16-byte aligned.
constexpr int kScanBatch = 8;
__global__ __launch_bounds__(kScanThreads) void radix_scan_kernel(uint32_t *hist, int64_t count) {
    __shared__ uint32_t wave_total[kScanThreads / 64];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t chunk = round_up(ceil_div(count, kScanThreads), 4);
    const int64_t a = min(t * chunk, count), b = min(a + chunk, count);
    const bool in_regs = chunk <= 4 * kScanBatch;   // uniform
    u32x4 *h4 = (u32x4 *)hist;
    u32x4 v[kScanBatch];
    uint32_t sum = 0;
    for (int64_t i = a; i < b; i += 4 * kScanBatch) {   // one trip when in_regs
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u)
            v[u] = i + 4 * u < b ? h4[(i >> 2) + u] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) sum += v[u][0] + v[u][1] + v[u][2] + v[u][3];
    }
    uint32_t incl = sum;   // inclusive scan of the chunk sums within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t up = __shfl_up(incl, o);
        if (lane >= o) incl += up;
    }
    if (lane == 63) wave_total[wave] = incl;
    __syncthreads();
    uint32_t run = incl - sum;   // exclusive prefix of this chunk
    for (int w = 0; w < wave; ++w) run += wave_total[w];
    for (int64_t i = a; i < b; i += 4 * kScanBatch) {
        if (!in_regs) {
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u)
                v[u] = i + 4 * u < b ? h4[(i >> 2) + u] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) {
            u32x4 o;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                o[c] = run;
                run += v[u][c];
            }
            if (i + 4 * u < b) h4[(i >> 2) + u] = o;
        }
    }
}

// Stable scatter of one pass.  Within a wave, the lanes holding the same digit are
// found with eight ballots (one per digit bit); a lane's rank is the number of those
// lanes below it.  Per-(round, wave) digit counts, prefix-summed in LDS in element
// order, give each group's offset inside the tile; the scanned counts give the tile's
// offset for the digit.
__global__ __launch_bounds__(kSortThreads) void radix_scatter_kernel(KeySource src, int64_t n,
                                                                     int shift,
                                                                     const uint32_t *scanned,
                                                                     int nblk, uint32_t *keys_out,
                                                                     uint32_t *vals_out) {
    __shared__ uint32_t seg[kSortSegs][kRadix];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    for (int i = t; i < kSortSegs * kRadix; i += kSortThreads) (&seg[0][0])[i] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kSortTile;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t key[kSortRounds], digit[kSortRounds], rank[kSortRounds];
#pragma unroll
    for (int r = 0; r < kSortRounds; ++r) {
        const int64_t e = base + r * kSortThreads + t;
        const bool valid = e < n;
        key[r] = valid ? src.key(e) : 0u;
        digit[r] = (key[r] >> shift) & (kRadix - 1);
        uint64_t same = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < kRadixBits; ++bit) {
            const uint64_t ones = __ballot(valid && ((digit[r] >> bit) & 1u));
            same &= ((digit[r] >> bit) & 1u) ? ones : ~ones;
        }
        rank[r] = (uint32_t)__popcll(same & below);
        if (valid && rank[r] == 0) seg[r * kSortWaves + wave][digit[r]] = (uint32_t)__popcll(same);
    }
    __syncthreads();
    if (t < kRadix) {   // exclusive prefix over the groups, per digit, in element order
        uint32_t run = 0;
        for (int g = 0; g < kSortSegs; ++g) {
            const uint32_t c = seg[g][t];
            seg[g][t] = run;
            run += c;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kSortRounds; ++r) {
        const int64_t e = base + r * kSortThreads + t;
        if (e < n) {
            const uint32_t pos = scanned[(int64_t)digit[r] * nblk + blockIdx.x] +
                                 seg[r * kSortWaves + wave][digit[r]] + rank[r];
            keys_out[pos] = key[r];
            vals_out[pos] = src.val(e);
        }
    }
}

__device__ __forceinline__ void add_bf16x8(float (&acc)[8], u32x4 v) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc[2 * q] += __builtin_bit_cast(float, v[q] << 16);
        acc[2 * q + 1] += __builtin_bit_cast(float, v[q] & 0xFFFF0000u);
    }
}

__device__ __forceinline__ void add_to_row(float *dst, const float (&acc)[8]) {
    f32x4 a = *(f32x4 *)dst, b = *(f32x4 *)(dst + 4);
    a += f32x4{acc[0], acc[1], acc[2], acc[3]};
    b += f32x4{acc[4], acc[5], acc[6], acc[7]};
    *(f32x4 *)dst = a;
    *(f32x4 *)(dst + 4) = b;
}

__device__ __forceinline__ void store_row(float *dst, const float (&acc)[8]) {
    *(f32x4 *)dst = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *(f32x4 *)(dst + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

// Block (b, cb): sorted positions [b kSegRows, ...) and columns [cb kSegCols, ...).
// Control flow depends only on the keys, which every thread reads from LDS, so it is
// uniform; a thread past h only skips its loads and stores.  Whether position q ends a
// row, and how, follows from the keys alone (sorted: the row began before the block
// exactly when its key equals the key just before the block), so each batch issues the
// loads of its dout rows and of the dw rows it finishes together.
// sk holds the keys of positions p0-1 .. p1 (vs where outside [0, n)), sv the tokens.
__device__ __forceinline__ void segment_block(
    int64_t b, int64_t cb, const uint32_t *__restrict__ keys, const uint32_t *__restrict__ vals,
    int64_t n, uint32_t vs, const uint16_t *__restrict__ dout, int64_t h, float *__restrict__ dw,
    float *__restrict__ part_first, float *__restrict__ part_last, uint32_t *sk, uint32_t *sv) {
    const int t = threadIdx.x;
    const int64_t p0 = b * kSegRows, p1 = min(p0 + kSegRows, n);
    const int rows = (int)(p1 - p0);
    for (int i = t; i < kSegRows + 2; i += kSegThreads) {
        const int64_t p = p0 - 1 + i;
        sk[i] = (p >= 0 && p < n) ? keys[p] : vs;
    }
    for (int i = t; i < rows; i += kSegThreads) sv[i] = vals[p0 + i];
    __syncthreads();
    if (sk[1] == vs) return;   // only off-shard tokens from here on
    const int64_t col = cb * kSegCols + 8 * t;
    const bool active = col < h;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int q0 = 0; q0 < rows; q0 += kSegBatch) {
        u32x4 v[kSegBatch];
        f32x4 d[kSegBatch][2];
#pragma unroll
        for (int u = 0; u < kSegBatch; ++u) {
            const int q = min(q0 + u, rows - 1);
            const uint32_t key = sk[q + 1], next = sk[q + 2];
            const bool ends = q + 1 == rows || next != key;
            const bool direct = ends && key != vs && key != sk[0] && !(q + 1 == rows && next == key);
            v[u] = active ? *(const u32x4 *)(dout + (int64_t)sv[q] * h + col) : u32x4{0u, 0u, 0u, 0u};
            if (active && direct && q0 + u < rows) {
                d[u][0] = *(const f32x4 *)(dw + (int64_t)key * h + col);
                d[u][1] = *(const f32x4 *)(dw + (int64_t)key * h + col + 4);
            }
        }
#pragma unroll
        for (int u = 0; u < kSegBatch; ++u) {
            const int q = q0 + u;
            if (q >= rows) break;
            const uint32_t key = sk[q + 1];
            if (key == vs) return;   // the rest are off-shard; nothing is pending
            add_bf16x8(acc, v[u]);
            const uint32_t next = sk[q + 2];
            if (next == key && q + 1 < rows) continue;   // the row goes on inside the block
            const bool before = sk[0] == key;
            const bool after = next == key;              // only possible at the block's end
            if (active) {
                if (!before && !after) {
                    d[u][0] += f32x4{acc[0], acc[1], acc[2], acc[3]};
                    d[u][1] += f32x4{acc[4], acc[5], acc[6], acc[7]};
                    *(f32x4 *)(dw + (int64_t)key * h + col) = d[u][0];
                    *(f32x4 *)(dw + (int64_t)key * h + col + 4) = d[u][1];
                } else if (before) {
                    store_row(part_first + b * h + col, acc);
                } else {
                    store_row(part_last + b * h + col, acc);
                }
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] = 0.f;
        }
    }
}

// One wave per (block of sorted positions, column block), the column block varying
// fastest: owned keys sort first, so the blocks with work are the first ones dispatched
// and run side by side, instead of each column block's few active waves being spread
// among the many that find only off-shard keys and return.  Grid-stride beyond the grid.
__global__ __launch_bounds__(kSegThreads) void segment_sum_kernel(
    const uint32_t *__restrict__ keys, const uint32_t *__restrict__ vals, int64_t n, uint32_t vs,
    const uint16_t *__restrict__ dout, int64_t h, float *__restrict__ dw,
    float *__restrict__ part_first, float *__restrict__ part_last, int64_t ncb, int64_t total) {
    __shared__ uint32_t sk[kSegRows + 2];
    __shared__ uint32_t sv[kSegRows];
    for (int64_t id = blockIdx.x; id < total; id += gridDim.x) {
        segment_block(id / ncb, id % ncb, keys, vals, n, vs, dout, h, dw, part_first, part_last,
                      sk, sv);
        __syncthreads();   // sk and sv are restaged by the next block
    }
}

// Rows that cross block edges: the block where such a row starts (its last row goes
// on into the next block, and did not come from the previous one) adds the row's
// pieces in block order, then adds the total to dw.  One workgroup per block; most
// blocks have no such row and return after reading three keys.  The blocks the row
// reaches into are contiguous (the keys are sorted), so the workgroup counts them with
// one boundary test per thread, then sums their pieces with independent loads.
constexpr int kFixThreads = 256;
constexpr int kFixBatch = 8;
__global__ __launch_bounds__(kFixThreads) void segment_fixup_kernel(
    const uint32_t *__restrict__ keys, int64_t n, uint32_t vs, int64_t h, float *__restrict__ dw,
    const float *__restrict__ part_first, const float *__restrict__ part_last) {
    const int64_t b = blockIdx.x;
    const int64_t p0 = b * kSegRows, p1 = min(p0 + kSegRows, n);
    if (p1 >= n) return;
    // the three boundary keys are loaded together: one memory latency for the many
    // blocks that return here
    const uint32_t key = keys[p1 - 1], next = keys[p1], prev = p0 > 0 ? keys[p0 - 1] : vs;
    if (key == vs || next != key) return;               // no row goes on past this block
    if (prev == key) return;                            // it started in an earlier block
    // m = number of following blocks that start with this row's key
    int64_t m = 0;
    for (;;) {
        const int64_t q = (b + 1 + m + threadIdx.x) * kSegRows;
        const int c = __syncthreads_count(q < n && keys[q] == key);
        m += c;
        if (c < kFixThreads) break;
    }
    for (int64_t col = 8 * threadIdx.x; col < h; col += 8 * kFixThreads) {
        f32x4 lo = *(const f32x4 *)(part_last + b * h + col);
        f32x4 hi = *(const f32x4 *)(part_last + b * h + col + 4);
        for (int64_t j0 = 1; j0 <= m; j0 += kFixBatch) {
            f32x4 a[kFixBatch], c[kFixBatch];
#pragma unroll
            for (int u = 0; u < kFixBatch; ++u) {
                const int64_t j = min(j0 + u, m);
                a[u] = *(const f32x4 *)(part_first + (b + j) * h + col);
                c[u] = *(const f32x4 *)(part_first + (b + j) * h + col + 4);
            }
#pragma unroll
            for (int u = 0; u < kFixBatch; ++u)
                if (j0 + u <= m) {
                    lo += a[u];
                    hi += c[u];
                }
        }
        const float acc[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        add_to_row(dw + (int64_t)key * h + col, acc);
    }
}

int radix_passes(int64_t vs) {   // digits needed for keys 0 .. vs (vs = off-shard)
    int bits = 0;
    while (bits < 32 && (vs >> bits) != 0) ++bits;
    return (int)ceil_div(bits > 0 ? bits : 1, kRadixBits);
}

}  // namespace

EmbedBwdWorkspace embed_bwd_workspace(int64_t n, int64_t h) {
    EmbedBwdWorkspace w;
    w.nblk = ceil_div(n, kSortTile);
    w.nseg = ceil_div(n, kSegRows);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (size_t)round_up((int64_t)bytes, 256);
        return o;
    };
    for (int i = 0; i < 2; ++i) {
        w.off_keys[i] = take((size_t)n * 4);
        w.off_vals[i] = take((size_t)n * 4);
    }
    w.off_hist = take((size_t)kRadix * w.nblk * 4);
    w.off_first = take((size_t)w.nseg * h * 4);
    w.off_last = take((size_t)w.nseg * h * 4);
    w.bytes = off;
    return w;
}

hipError_t launch_embed_bwd(const int64_t *ids, int64_t n, const uint16_t *dout, int64_t start,
                            int64_t vs, int64_t h, float *dw, void *ws, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const EmbedBwdWorkspace w = embed_bwd_workspace(n, h);
    char *base = (char *)ws;
    uint32_t *keys[2] = {(uint32_t *)(base + w.off_keys[0]), (uint32_t *)(base + w.off_keys[1])};
    uint32_t *vals[2] = {(uint32_t *)(base + w.off_vals[0]), (uint32_t *)(base + w.off_vals[1])};
    uint32_t *hist = (uint32_t *)(base + w.off_hist);
    const int nblk = (int)w.nblk;
    const int passes = radix_passes(vs);
    for (int p = 0; p < passes; ++p) {
        KeySource src{ids, p == 0 ? nullptr : keys[(p - 1) & 1], p == 0 ? nullptr : vals[(p - 1) & 1],
                      start, (uint32_t)vs};
        hipLaunchKernelGGL(radix_count_kernel, dim3(nblk), dim3(kSortThreads), 0, stream, src, n,
                           p * kRadixBits, hist, nblk);
        hipLaunchKernelGGL(radix_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, hist,
                           (int64_t)kRadix * nblk);
        hipLaunchKernelGGL(radix_scatter_kernel, dim3(nblk), dim3(kSortThreads), 0, stream, src, n,
                           p * kRadixBits, hist, nblk, keys[p & 1], vals[p & 1]);
    }
    const uint32_t *sk = keys[(passes - 1) & 1], *sv = vals[(passes - 1) & 1];
    float *first = (float *)(base + w.off_first), *last = (float *)(base + w.off_last);
    const int64_t ncb = ceil_div(h, kSegCols), total = w.nseg * ncb;
    hipLaunchKernelGGL(segment_sum_kernel, dim3((unsigned)std::min<int64_t>(total, kSegMaxGrid)),
                       dim3(kSegThreads), 0, stream, sk, sv, n, (uint32_t)vs, dout, h, dw, first,
                       last, ncb, total);
    hipLaunchKernelGGL(segment_fixup_kernel, dim3((unsigned)w.nseg), dim3(kFixThreads), 0, stream, sk,
                       n, (uint32_t)vs, h, dw, first, last);
    return hipGetLastError();
}

}  // namespace vp
