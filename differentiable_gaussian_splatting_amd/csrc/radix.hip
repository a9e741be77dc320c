// radix.hip -- stable LSD radix sort of (u32 key, u32 value) pairs.
//
// Each pass takes at most 8 key bits (the passes share them evenly), or a
// single pass takes up to 10 bits: a per-block digit histogram (LDS atomics) laid out
// digit-major (digit * n_blocks + block), an exclusive scan of each digit's
// row with its total (one workgroup per digit), and a stable scatter, whose
// blocks add the scan of the digit totals.  The scatter ranks a
// block's elements in element order: 256 elements per round, a wavefront
// finds the lanes holding the same digit with one ballot per digit bit
// (lane rank = popcount of same-digit lanes below it), per-wave digit counts
// go through LDS, and a running per-digit base carries the order across
// rounds.  Stable passes make the result sorted by the whole key with ties in
// input order.
#include "gs_device.h"
#include "gs_internal.h"

namespace {

constexpr int kRB = 256;      // threads per block
constexpr int kRItems = 8;    // rounds (elements per thread)
constexpr int kRTile = kRB * kRItems;

template <int kRadix>
__global__ __launch_bounds__(kRB) void k_radix_hist(const uint32_t* __restrict__ keys, int64_t n, int shift,
                                                    uint32_t mask, uint32_t* __restrict__ hist, int64_t nb)
{
    __shared__ uint32_t h[kRadix];
    for (int d = threadIdx.x; d < kRadix; d += kRB) h[d] = 0u;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kRTile;
    uint32_t kk[kRItems];   // all of the thread's keys requested before the first count
#pragma unroll
    for (int r = 0; r < kRItems; ++r) {
        const int64_t i = base + (int64_t)r * kRB + threadIdx.x;
        kk[r] = i < n ? keys[i] : 0u;
    }
#pragma unroll
    for (int r = 0; r < kRItems; ++r)
        if (base + (int64_t)r * kRB + threadIdx.x < n) atomicAdd(&h[(kk[r] >> shift) & mask], 1u);
    __syncthreads();
    for (int d = threadIdx.x; d <= (int)mask; d += kRB) hist[(int64_t)d * nb + blockIdx.x] = h[d];
}

__device__ __forceinline__ uint32_t block_excl_scan256(uint32_t v, uint32_t* sh)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t u = __shfl_up(x, o, 64);
        if (lane >= o) x += u;
    }
    if (lane == 63) sh[wave] = x;
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w) before += sh[w];
    __syncthreads();
    return before + x - v;
}

// Per digit (one workgroup of kDSW wavefronts): exclusive scan of its row of
// per-block counts (the histogram is digit-major, so a row is contiguous), in
// place, and the digit's total.  Each wavefront owns 1/kDSW of the row: it
// sums it in coalesced chunks, then rescans it chunk by chunk with a carry.
// With only 2^bits rows, the rescans' chains of dependent 64-entry chunks set
// the time, hence many wavefronts per row.
constexpr int kDSW = 16;
__global__ __launch_bounds__(64 * kDSW) void k_radix_digit_scan(uint32_t* __restrict__ hist, int64_t nb,
                                                                uint32_t* __restrict__ dtot)
{
    __shared__ uint32_t wsum[kDSW];
    uint32_t* row = hist + (int64_t)blockIdx.x * nb;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t seg = ((nb + kDSW - 1) / kDSW + 63) / 64 * 64;
    const int64_t t0 = min(nb, (int64_t)wave * seg), t1 = min(nb, t0 + seg);
    uint64_t s = 0;
    for (int64_t c = t0; c < t1; c += 256) {
        uint32_t a[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) a[u] = c + 64 * u + lane < t1 ? row[c + 64 * u + lane] : 0u;
        s += (uint64_t)a[0] + a[1] + a[2] + a[3];
    }
    s = gsd::wave_sum_u64(s);
    if (lane == 0) wsum[wave] = (uint32_t)s;
    __syncthreads();
    uint32_t carry = 0;
    for (int w = 0; w < wave; ++w) carry += wsum[w];
    for (int64_t c = t0; c < t1; c += 64) {
        const uint32_t v = c + lane < t1 ? row[c + lane] : 0u;
        uint32_t x = v;
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t u = (uint32_t)__shfl_up((int)x, d, 64);
            if (lane >= d) x += u;
        }
        if (c + lane < t1) row[c + lane] = carry + x - v;
        carry += (uint32_t)__shfl((int)x, 63, 64);
    }
    if (threadIdx.x == 0) {
        uint32_t tot = 0;
        for (int w = 0; w < kDSW; ++w) tot += wsum[w];
        dtot[blockIdx.x] = tot;
    }
}

// Stable scatter of one block's kRTile elements: (1) local ranks in element
// order, (2) the block's elements placed digit-sorted in LDS, (3) written out
// digit run by digit run, so that consecutive lanes write consecutive
// addresses.  Ranks, round by round (kRB elements each): a wavefront's lanes
// with equal digits are found with one ballot per digit bit; the first lane
// of each such group records the group size in wh[wave][digit] tagged with
// the round (entries with another tag count as zero, so wh is cleared only
// once), and after the round the group sizes are added to run[digit] with one
// LDS atomic per (wavefront, digit).  Two barriers per round: one after the
// tagged sizes are written, one after every lane has read run[].
template <int kRadix>
__global__ __launch_bounds__(kRB) void k_radix_scatter(const uint32_t* __restrict__ kin,
                                                       const uint32_t* __restrict__ vin, int64_t n, int shift,
                                                       int bits, const uint32_t* __restrict__ hpre,
                                                       const uint32_t* __restrict__ dtot, int64_t nb,
                                                       uint32_t* __restrict__ kout, uint32_t* __restrict__ vout,
                                                       uint64_t* __restrict__ digit_off, int n_seg)
{
    __shared__ uint32_t run[kRadix];
    __shared__ uint32_t lstart[kRadix];
    __shared__ uint32_t gbase[kRadix];
    __shared__ uint32_t wh[kRB / 64][kRadix];   // (round + 1) << 16 | group size
    __shared__ uint32_t sk[kRTile];
    __shared__ uint32_t sv[kRTile];
    __shared__ uint32_t scan_sh[kRB / 64];
    const uint32_t mask = (1u << bits) - 1u;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t lt = (1ull << lane) - 1ull;
    for (int d = threadIdx.x; d < kRadix; d += kRB) run[d] = 0u;
    // output base of each digit for this block: the digit's start (exclusive
    // scan of the digit totals; digits above the mask are empty) plus the
    // earlier blocks' count of it.  A single pass over keys < n_seg also
    // reports where each digit's run starts, and the total.
    {
        constexpr int P = kRadix / kRB;
        uint32_t t[P];
        uint32_t part = 0;
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const int d = threadIdx.x * P + q;
            t[q] = (uint32_t)d <= mask ? dtot[d] : 0u;
            part += t[q];
        }
        uint32_t at = block_excl_scan256(part, scan_sh);
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const int d = threadIdx.x * P + q;
            gbase[d] = at + ((uint32_t)d <= mask ? hpre[(int64_t)d * nb + blockIdx.x] : 0u);
            if (digit_off && blockIdx.x == 0 && d < n_seg) digit_off[d] = at;
            at += t[q];
        }
        if (digit_off && blockIdx.x == 0 && threadIdx.x == 0) digit_off[n_seg] = (uint64_t)n;
    }
    for (int q = threadIdx.x; q < (kRB / 64) * kRadix; q += kRB) (&wh[0][0])[q] = 0u;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kRTile;
    uint32_t kk[kRItems], vv[kRItems], ll[kRItems], dd[kRItems];
    // every element of the thread is requested before the first round
#pragma unroll
    for (int r = 0; r < kRItems; ++r) {
        const int64_t i = base + (int64_t)r * kRB + threadIdx.x;
        kk[r] = i < n ? kin[i] : 0u;
        vv[r] = i < n ? vin[i] : 0u;
    }
#pragma unroll
    for (int r = 0; r < kRItems; ++r) {
        const int64_t i = base + (int64_t)r * kRB + threadIdx.x;
        const bool valid = i < n;
        const uint32_t key = kk[r];
        const uint32_t d = valid ? (key >> shift) & mask : 0u;
        uint64_t peers = gsd::ballot(valid);
        for (int b = 0; b < bits; ++b) {
            const uint64_t bb = gsd::ballot(valid && ((d >> b) & 1u));
            peers &= ((d >> b) & 1u) ? bb : ~bb;
        }
        const uint32_t rank = (uint32_t)__popcll(peers & lt);
        const uint32_t size = (uint32_t)__popcll(peers);
        const uint32_t tag = (uint32_t)(r + 1) << 16;
        if (valid && rank == 0) wh[wave][d] = tag | size;
        __syncthreads();                       // tagged group sizes of the round written
        uint32_t loc = run[d] + rank;
        for (int w = 0; w < wave; ++w) {
            const uint32_t t = wh[w][d];
            loc += (t & 0xFFFF0000u) == tag ? (t & 0xFFFFu) : 0u;
        }
        dd[r] = valid ? d : 0xFFFFFFFFu;
        ll[r] = loc;
        __syncthreads();                       // every lane has read run[] for the round
        if (valid && rank == 0) atomicAdd(&run[d], size);
    }
    __syncthreads();
    // local start of every digit run (each thread scans kRadix / kRB
    // consecutive digits)
    {
        constexpr int P = kRadix / kRB;
        uint32_t part = 0;
#pragma unroll
        for (int q = 0; q < P; ++q) part += run[threadIdx.x * P + q];
        uint32_t at = block_excl_scan256(part, scan_sh);
#pragma unroll
        for (int q = 0; q < P; ++q) {
            lstart[threadIdx.x * P + q] = at;
            at += run[threadIdx.x * P + q];
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kRItems; ++r)
        if (dd[r] != 0xFFFFFFFFu) {
            const uint32_t pos = lstart[dd[r]] + ll[r];
            sk[pos] = kk[r];
            sv[pos] = vv[r];
        }
    __syncthreads();
    const int nvalid = (int)min<int64_t>(kRTile, n - base);
    for (int q = threadIdx.x; q < nvalid; q += kRB) {
        const uint32_t key = sk[q];
        const uint32_t d = (key >> shift) & mask;
        const uint32_t o = gbase[d] + (uint32_t)q - lstart[d];
        kout[o] = key;
        vout[o] = sv[q];
    }
}

}  // namespace

// Sorts n pairs by the low key_bits bits of the keys (stable).  k0/v0 hold the
// input; k1/v1 are scratch of the same size.  *in_second is set when the
// sorted result ends in (k1, v1).  Offsets of one pass fit u32: n < 2^32.
// digit_off (optional, n_seg + 1 entries): when the sort takes a single pass
// and every key's low bits are < n_seg, the first output position of each
// value s in [0, n_seg) and the total are written there, and *off_written is
// set.  scratch (optional, radix_scratch_words(n) u32): the histogram and
// digit totals; without it the sort allocates them on ctx->stream.
int64_t radix_scratch_words(int64_t n)
{
    return 1024 * ceil_div(std::max<int64_t>(n, 1), kRTile) + 1024;
}

gs_status launch_radix_sort(gs_ctx* ctx, uint32_t* k0, uint32_t* v0, uint32_t* k1, uint32_t* v1, int64_t n,
                            int key_bits, bool* in_second, uint64_t* digit_off, int64_t n_seg, bool* off_written,
                            uint32_t* scratch)
{
    *in_second = false;
    if (off_written) *off_written = false;
    if (n <= 1 || key_bits <= 0) return GS_OK;
    if (n >= (1ll << 32)) return gs_fail(ctx, GS_ERR_OVERFLOW, "radix sort of %lld >= 2^32 pairs", (long long)n);
    const int64_t nb = ceil_div(n, kRTile);
    // up to 10 bits in one pass, else 8-bit passes
    const bool wide = key_bits <= 10;
    const int radix = wide ? 1024 : 256;
    std::vector<GsAlloc> tmp;
    uint32_t* hist = scratch ? scratch
                             : (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * radix * nb, GS_MEM_SCRATCH, &tmp);
    uint32_t* dtot = scratch ? scratch + 1024 * nb
                             : (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * radix, GS_MEM_SCRATCH, &tmp);
    if (!hist || !dtot) {
        gs_free_all(ctx, &tmp);
        return GS_ERR_OOM;
    }
    gs_status st = GS_OK;
    uint32_t *ki = k0, *vi = v0, *ko = k1, *vo = v1;
    // 8-bit passes share the bits evenly (13 bits: 7 + 6, not 8 + 5): a
    // block's elements land in one run per digit present, and with 2^8
    // digits over a block of 2048 those runs average 8 elements, too short
    // for whole-line writes
    const int n_pass = wide ? 1 : (key_bits + 7) / 8;
    const int step = wide ? key_bits : (key_bits + n_pass - 1) / n_pass;
    const bool want_off = digit_off && off_written && wide && n_seg >= 0 && n_seg <= radix;
    for (int shift = 0; shift < key_bits && st == GS_OK; shift += step) {
        const int bits = std::min(step, key_bits - shift);
        const uint32_t mask = (1u << bits) - 1u;
        {
            GsTimerScope ts(ctx, "radix");
            if (wide)
                hipLaunchKernelGGL(k_radix_hist<1024>, dim3((unsigned)nb), dim3(kRB), 0, ctx->stream, ki, n, shift,
                                   mask, hist, nb);
            else
                hipLaunchKernelGGL(k_radix_hist<256>, dim3((unsigned)nb), dim3(kRB), 0, ctx->stream, ki, n, shift,
                                   mask, hist, nb);
        }
        {
            // per digit that can occur: its row of block counts scanned in
            // place, and its total
            GsTimerScope ts(ctx, "radix");
            hipLaunchKernelGGL(k_radix_digit_scan, dim3(mask + 1u), dim3(64 * kDSW), 0, ctx->stream, hist, nb, dtot);
        }
        {
            GsTimerScope ts(ctx, "radix");
            if (wide)
                hipLaunchKernelGGL(k_radix_scatter<1024>, dim3((unsigned)nb), dim3(kRB), 0, ctx->stream, ki, vi, n,
                                   shift, bits, hist, dtot, nb, ko, vo, want_off ? digit_off : nullptr, (int)n_seg);
            else
                hipLaunchKernelGGL(k_radix_scatter<256>, dim3((unsigned)nb), dim3(kRB), 0, ctx->stream, ki, vi, n,
                                   shift, bits, hist, dtot, nb, ko, vo, nullptr, 0);
        }
        std::swap(ki, ko);
        std::swap(vi, vo);
        *in_second = !*in_second;
    }
    gs_free_all(ctx, &tmp);
    if (st != GS_OK) return st;
    GS_HIP(ctx, hipGetLastError());
    if (want_off) *off_written = true;
    return GS_OK;
}
