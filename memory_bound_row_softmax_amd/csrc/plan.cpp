// plan.cpp -- host planner (no HIP).
//
// The QuACK article (无需CUDA代码，给H100加速33%-50%) chooses, before launch, how
// threads map onto the reduction dimension (section 硬件感知的加载与存储策略, the
// thread-value layout) and whether a row is reduced inside one block or across a
// cluster of blocks, depending on the size of the reduction dimension (section
// 硬件感知的归约策略, the last paragraph).  It also notes that the tuning is per
// operator and per shape (section 总结).  This file is that choice for gfx950:
//   * a row of up to P * R elements lives in the registers of R lanes
//     (R <= 64: part of one wave; R > 64: R / 64 waves joined through LDS);
//   * longer rows are split over G workgroups that exchange partial results
//     through global memory (the cluster / distributed-shared-memory level of
//     the pages has no counterpart on this GPU);
//   * cross-entropy writes no per-element output, so it streams its row with a
//     running (max, sum) instead of holding it.
#include "plan.hpp"

#include <atomic>

#include "configs.hpp"

namespace rr {

// The test overrides.  Each field is read with one relaxed load per call; `active`
// lets a call that sees no override skip the rest.
namespace {
std::atomic<bool> g_active{false};
std::atomic<int> g_kind{0}, g_P{0}, g_R{0}, g_G{0}, g_groups{0}, g_spin{0};
}  // namespace

void set_test_overrides(const TestOverrides &o) {
    g_kind.store(o.kind, std::memory_order_relaxed);
    g_P.store(o.P, std::memory_order_relaxed);
    g_R.store(o.R, std::memory_order_relaxed);
    g_G.store(o.G, std::memory_order_relaxed);
    g_groups.store(o.groups, std::memory_order_relaxed);
    g_spin.store(o.spin, std::memory_order_relaxed);
    const bool any = o.kind || o.P || o.R || o.G || o.groups || o.spin;
    g_active.store(any, std::memory_order_release);
}

TestOverrides test_overrides() {
    TestOverrides o;
    if (!g_active.load(std::memory_order_acquire)) return o;
    o.kind = g_kind.load(std::memory_order_relaxed);
    o.P = g_P.load(std::memory_order_relaxed);
    o.R = g_R.load(std::memory_order_relaxed);
    o.G = g_G.load(std::memory_order_relaxed);
    o.groups = g_groups.load(std::memory_order_relaxed);
    o.spin = g_spin.load(std::memory_order_relaxed);
    return o;
}

static int cfg_op(int op) {
    switch (op) {
    case kOpSoftmax: return kCfgSoftmax;
    case kOpXentGrad: return kCfgXentGrad;
    case kOpSoftmaxBwd: return kCfgSoftmaxBwd;
    default: return kCfgRmsnorm;
    }
}
static int elem_bytes(int dtype) { return dtype == kBf16 ? 2 : 4; }

bool block_config_ok(int op, int dtype, bool vec, int P, int R) {
#define RR_X(p, r) \
    if (P == p && R == r) return block_config_enabled(cfg_op(op), elem_bytes(dtype), vec, p, r);
    RR_BLOCK_CONFIGS(RR_X)
#undef RR_X
    return false;
}

bool stream_config_ok(int op, int dtype, bool vec, int P, int R, int G) {
    if (P == kPackedP) {  // packed bf16: RMSNorm forward, 128-bit path
        if (dtype != kBf16 || !vec || op != kOpRmsnorm) return false;
#define RR_X(r, g) \
    if (R == r && G == g) return true;
        RR_PACKED_CONFIGS(RR_X)
#undef RR_X
        return false;
    }
#define RR_X(p, r, g)                    \
    if (P == p && R == r && G == g)      \
        return stream_config_enabled(cfg_op(op), elem_bytes(dtype), vec, p, r, g);
    RR_STREAM_CONFIGS(RR_X)
#undef RR_X
    return false;
}

bool xent_config_exists(int P, int R) {
#define RR_X(p, r) \
    if (P == p && R == r) return true;
    RR_XENT_CONFIGS(RR_X)
#undef RR_X
    return false;
}

bool rmsbwd_config_ok(int dtype, bool vec, int P, int R, int G) {
#define RR_X(p, r, g) \
    if (P == p && R == r && G == g) return rmsbwd_config_enabled(vec, p, elem_bytes(dtype));
    RR_RMSBWD_CONFIGS(RR_X)
#undef RR_X
    return false;
}

size_t grid_ws_bytes(int G, int64_t M) {
    int64_t groups = M < max_groups_for(G) ? M : max_groups_for(G);
    if (groups < 1) groups = 1;
    return (size_t)kWsHeader + (size_t)groups * (size_t)group_stride_for(G);
}

static int64_t next_pow2(int64_t v) {
    int64_t p = 1;
    while (p < v) p <<= 1;
    return p;
}

static void fill_geometry(Plan *p) {
    p->block = block_threads_for(p->R);
    p->rows_per_block = rows_per_block_for(p->R);
}

// Default row-resident choice: a table of the fastest configuration measured on
// MI355X for each op, dtype and power-of-four N (16384 rows, every compiled
// configuration timed, cold HBM reads), applied to the smallest tabulated N
// that is >= the call's N, then narrowed to the fewest lanes (block) or
// workgroups (stream) that still hold the row.  Patterns behind the numbers:
// short rows prefer two 16-byte chunks per lane and many lanes (more waves,
// fewer loads in flight per wave); long rows prefer the persistent stream
// kernels, whose second register buffer keeps the next row's loads in flight
// while a row is reduced, with as few workgroups per row as fit (each extra one
// joins the exchange).  Differences between the top few configurations are a
// few percent.  The softmax and RMSNorm forward entries from 32768 to 1048576
// elements were measured again after the split rows took granule-interleaved
// shares (configs.hpp, split_granule) and bf16 kernels two workgroups per CU
// (stream_waves): GB/s averaged over six byte offsets between input and output,
// since a single placement can be off by up to 10 %.  64 values on 256 lanes then
// led from 32768 to 131072 elements (fp32 softmax at 131072: 6460 against 6015 GB/s
// for 64 x 512 on 4 workgroups, whose rate also swung from 5628 to 6240 with the
// offset), and the fp32 RMSNorm at 262144 took 64 x 512 on 8 (6626 against 5774).
// The softmax backward and the cross-entropy gradient were measured the same way
// (the gradient's bf16 rows of 131072: 5373 against 4478 GB/s), and the fp32 softmax
// and RMSNorm at 16384 took 16 values on a 1024-lane stream workgroup (6188 against
// 5490 GB/s for 64 x 512, whose lanes were half empty; RMSNorm 6340 against 5953 for
// the 16 x 1024 block kernel; bf16 RMSNorm 6026 against 5456 for 32 x 1024).
struct Choice {
    bool stream;
    int P, R, G;
};
constexpr int kTunedBuckets = 17;
constexpr int64_t kTunedN[kTunedBuckets] = {256,    1024,    4096,    5120,    6144,   8192,
                                            12288,  16384,   32768,   65536,   131072, 262144,
                                            524288, 1048576, 2097152, 4194304, 8388608};
// A choice with P = 0: no on-chip plan (softmax and RMSNorm then read the row twice).
constexpr Choice kTwoReads = {false, 0, 0, 0};
//   [op: softmax, rmsnorm, softmax backward, cross-entropy gradient][dtype: f32, bf16][N bucket]
// (the four longest buckets were timed at 4096, 2048, 512-1024 and 256-512 rows; the
// 5120, 6144, 8192 and 12288 buckets were added later, where the plans interpolated
// from their neighbours ran 3-37 % slower; at 5120, 6144 and 12288 the softmax and
// RMSNorm were timed, at 12288 also the cross-entropy gradient, and the other
// entries there are the ones those lengths used before)
static const Choice kTuned[4][2][kTunedBuckets] = {
    {{{false, 16, 16, 1}, {false, 8, 128, 1}, {false, 8, 512, 1}, {false, 32, 256, 1},
      {false, 32, 256, 1}, {false, 64, 128, 1}, {false, 64, 256, 1}, {true, 16, 1024, 1},
      {true, 64, 256, 2}, {true, 64, 256, 4}, {true, 64, 256, 8}, {true, 64, 512, 8},
      {true, 64, 512, 16}, {true, 64, 512, 32}, {true, 64, 512, 64}, {true, 64, 512, 128},
      {true, 64, 512, 256}},
     {{false, 16, 16, 1}, {false, 16, 64, 1}, {false, 16, 256, 1}, {false, 32, 256, 1},
      {false, 32, 256, 1}, {false, 16, 512, 1}, {false, 64, 256, 1}, {false, 64, 256, 1},
      {true, 32, 1024, 1}, {true, 32, 512, 4}, {true, 64, 256, 8}, {true, 64, 512, 8},
      {true, 64, 512, 16}, {true, 64, 512, 32}, {true, 64, 512, 64}, {true, 64, 512, 128},
      {true, 64, 512, 256}}},
    {{{false, 16, 16, 1}, {false, 16, 64, 1}, {false, 8, 512, 1}, {false, 16, 512, 1},
      {false, 32, 256, 1}, {false, 64, 128, 1}, {false, 16, 1024, 1}, {true, 16, 1024, 1},
      {true, 64, 256, 2}, {true, 64, 256, 4}, {true, 64, 256, 8}, {true, 64, 512, 8},
      {true, 64, 512, 16}, {true, 64, 512, 32}, {true, 64, 512, 64}, {true, 64, 512, 128},
      {true, 64, 512, 256}},
     {{false, 16, 16, 1}, {false, 16, 64, 1}, {false, 8, 512, 1}, {false, 32, 256, 1},
      {false, 32, 256, 1}, {false, 16, 512, 1}, {false, 64, 256, 1}, {true, 16, 1024, 1},
      {true, 32, 512, 2}, {true, 32, 512, 4}, {true, 64, 256, 8}, {true, kPackedP, 256, 8},
      {true, kPackedP, 512, 8}, {true, kPackedP, 512, 16}, {true, kPackedP, 512, 32}, {true, kPackedP, 512, 64},
      {true, kPackedP, 512, 128}}},
    // softmax backward (y and dy both held: at most 32 values per lane in a stream kernel)
    {{{false, 16, 16, 1}, {false, 8, 128, 1}, {false, 16, 256, 1}, {false, 32, 256, 1},
      {false, 32, 256, 1}, {false, 32, 256, 1}, {false, 32, 1024, 1}, {false, 32, 1024, 1},
      {true, 16, 1024, 2}, {true, 32, 512, 4}, {true, 32, 512, 8}, {true, 16, 1024, 16},
      {true, 32, 512, 32}, {true, 32, 512, 64}, kTwoReads, kTwoReads, kTwoReads},
     {{false, 8, 32, 1}, {false, 8, 128, 1}, {false, 8, 512, 1}, {false, 16, 512, 1},
      {false, 16, 512, 1}, {false, 16, 512, 1}, {false, 16, 1024, 1}, {false, 16, 1024, 1},
      {true, 32, 512, 2}, {true, 32, 512, 4}, {true, 32, 512, 8}, {true, 32, 512, 16},
      {true, 32, 512, 32}, {true, 32, 512, 64}, kTwoReads, kTwoReads, kTwoReads}},
    // cross-entropy forward fused with its gradient (the softmax kernels; block kernels
    // hold longer rows here than for the softmax)
    {{{false, 16, 16, 1}, {false, 8, 128, 1}, {false, 8, 512, 1}, {false, 32, 256, 1},
      {false, 32, 256, 1}, {false, 32, 256, 1}, {false, 16, 1024, 1}, {true, 16, 1024, 1},
      {true, 64, 256, 2}, {true, 64, 256, 4}, {true, 64, 256, 8}, {true, 64, 256, 16},
      {true, 64, 512, 16}, {true, 64, 512, 32}, {true, 64, 512, 64}, kTwoReads, kTwoReads},
     {{false, 16, 16, 1}, {false, 64, 16, 1}, {false, 16, 256, 1}, {false, 32, 256, 1},
      {false, 32, 256, 1}, {false, 32, 256, 1}, {false, 64, 256, 1}, {false, 32, 512, 1},
      {false, 64, 512, 1}, {false, 64, 1024, 1}, {true, 64, 256, 8}, {true, 64, 256, 16},
      {true, 32, 1024, 16}, {true, 64, 512, 32}, {true, 64, 512, 64}, kTwoReads, kTwoReads}},
};

// Up to this many rows, a row that one workgroup of the stream kernels holds is
// not split: a persistent row group then has only a few rows, so the split row's
// exchange is no longer hidden behind the next rows' loads.  Measured on MI355X
// for fp32 rows of 32768 elements (softmax, M = 512 .. 4096): 5.67-5.92 TB/s on
// one workgroup of 32 values x 1024 lanes against 3.60-5.53 split over two; at
// 8192 rows and more the table's split plan is as fast or faster.
constexpr int64_t kFewRows = 4096;

// bf16 softmax rows split over 64 values x 512 lanes take exactly as many
// workgroups as the row needs when that is 3, 5 or 6 (compiled besides the powers
// of two) instead of the next power of two.  A lane runs every register through the
// exponential whether or not it holds an element, and at two bytes per element that
// work shows.  Measured on MI355X (bf16 softmax, 16384 rows): 151936 elements 5548
// GB/s on 5 workgroups against 4105 on 8, 70000 5089 on 3 against 4129 on 4, 180000
// 5261 on 6 against 4713 on 8.  Seven lost to eight (4892 against 5119 at 200000
// elements), which then deferred the exchange, so 7 is not compiled; eight now run
// two workgroups per CU without the deferral (5791 GB/s at 200000).  These plans
// replace whatever the table chose for the row (64 values on 256 lanes at 70000
// elements, after the re-measurement above: 4890 GB/s against 5177 on 64 x 512 x 3,
// offset-averaged); a row that needs 4 keeps the table's plan.
// fp32 softmax rows take 5 or 6 the same way (offset-averaged GB/s, exact against the
// table: 151936 elements 6155 on 5 against 5472 on 8, 163840 6134 against 5873,
// 180000 6189 on 6 against 5778); on 3 they gained at 70000 elements (+2 %) but lost
// at 98304 (-5 %), so fp32 keeps the table there.
// The bf16 cross-entropy gradient, whose 64 x 512 kernels need more than 128 VGPRs
// (one workgroup per CU), takes 64 values x 256 lanes on exactly ceil(N / 16384)
// workgroups from 3 to 16 (every count compiled; four workgroups per CU) for rows of
// 32769 to 262144 elements, whatever the table chose.  Offset-averaged GB/s, 16384
// rows, the previous plan -> this one: 40000 elements (block 64 x 1024) 4377 ->
// 5293 (on 3), 65536 (block) 5515 -> 6104 (4), 70000 (64 x 512 x 3) 3501 -> 5232
// (5), 100000 (64 x 256 x 8) 4240 -> 5369 (7), 151936 (64 x 512 x 5) 4073 -> 5450
// (10), 200000 (64 x 256 x 16) 3936 -> 5337 (13).  With few rows the split row
// still won over the block kernel (512 rows: 40000 elements 3730 -> 4880, 65536
// 5180 -> 5600; 256 rows of 151936: 3620 on 64 x 512 x 5 -> 5100).
static void exact_groups(int op, int dtype, bool vec, int64_t N, Plan *p) {
    if (!vec) return;
    if (op == kOpXentGrad && dtype == kBf16) {
        const int64_t need = (N + 64 * 256 - 1) / (64 * 256);
        if (need >= 3 && need <= 16 &&
            stream_config_ok(op, dtype, vec, 64, 256, (int)need)) {
            p->stream = true;
            p->P = 64;
            p->R = 256;
            p->G = (int)need;
        }
        return;
    }
    if (!p->stream || p->G <= 2) return;
    const bool bf16 = dtype == kBf16 && op == kOpSoftmax;
    const bool f32 = dtype != kBf16 && op == kOpSoftmax;
    if (!bf16 && !f32) return;
    const int64_t need = (N + 64 * 512 - 1) / (64 * 512);
    if (((bf16 && need == 3) || need == 5 || need == 6) &&
        stream_config_ok(op, dtype, vec, 64, 512, (int)need)) {
        p->P = 64;
        p->R = 512;
        p->G = (int)need;
    }
}

// Unaligned bf16 softmax and RMSNorm rows split over 2 to 8 workgroups take 32
// values on 512 lanes up to this many elements, 16 values on 1024 lanes beyond
// (same box, GB/s, 8192 rows, 16 -> 32 values: softmax 32001 3171 -> 3647, 50257
// 2691 -> 3554, 65537 2466 -> 2714, 100001 (RMSNorm) 3599 -> 3493, 151935 2582 ->
// 2506; RMSNorm 50257 3149 -> 3718).
constexpr int64_t kElemWideMaxN = 81920;

static bool try_choice(int op, int dtype, bool vec, int64_t N, Choice c, Plan *p) {
    if (c.stream) {
        if (!vec && c.P > 16 && N > kElemWideMaxN) return false;
        while (c.G > 1 && (int64_t)c.P * c.R * (c.G / 2) >= N) c.G /= 2;
        if ((int64_t)c.P * c.R * c.G < N || !stream_config_ok(op, dtype, vec, c.P, c.R, c.G))
            return false;
    } else {
        const int64_t r = next_pow2((N + c.P - 1) / c.P);
        c.R = r < 16 ? 16 : (int)(r > 4096 ? 4096 : r);
        if (c.R > 1024 || !block_config_ok(op, dtype, vec, c.P, c.R)) return false;
    }
    p->stream = c.stream;
    p->P = c.P;
    p->R = c.R;
    p->G = c.G;
    return true;
}


static bool default_row(int op, int dtype, bool vec, int64_t M, int64_t N, Plan *p) {
    const int o = op == kOpRmsnorm ? 1 : op == kOpSoftmaxBwd ? 2 : op == kOpXentGrad ? 3 : 0;
    const int d = dtype == kBf16 ? 1 : 0;
    int k = 0;
    while (k < kTunedBuckets - 1 && kTunedN[k] < N) ++k;
    if (N <= kTunedN[kTunedBuckets - 1]) {
        Choice c = kTuned[o][d][k];
        if (c.P == 0) return false;  // no on-chip plan measured faster than two reads
        // Softmax rows on 128 workgroups (2M to 4M elements) measured faster than
        // two reads only when they fill at least 9/10 of the plan: fp32 rows of
        // 3.5M, 3.67M, 3.9M and 4M elements ran at 0.94, 0.97, 1.03 and 1.10 times
        // the two-read rate.  RMSNorm gained at every fill measured (1.14-1.36).
        // Rows of 4M to 8M elements, on a workgroup of every CU (256, or 128 packed
        // bf16 RMSNorm workgroups), the same: offset-averaged GB/s, two reads -> on
        // chip, full rows (8388608): softmax fp32 4567 -> 6181, bf16 4646 -> 5528,
        // RMSNorm fp32 3499 -> 4622, bf16 4388 -> 5170 (before the RMSNorm deferred
        // its exchange; now 6224 and 6078-6127); at 9/10 (softmax fp32 7.6M) 4544
        // -> 6126; at 0.72 (6M) the fp32 softmax gained (4608 -> 5593) and the bf16
        // softmax lost (4673 -> 4024); at 0.54 both lost.  bf16
        // softmax rows of 1M to 2M elements on 64 workgroups likewise (1.5M: 4635 ->
        // 4285; 2M: 4911 -> 5550; 0.91 of 128 workgroups, 3.8M: 4735 -> 4876).
        // The RMSNorm, since it defers the exchange from 16 workgroups, gains at
        // every fill measured and is exempt: fp32 on 256 workgroups, 6M 4380 ->
        // 5422-5465, 4.5M 4307 -> 4652-4660; packed bf16 on 128, 6M 4473 -> 5374,
        // 4.5M 4141 -> 4680; on 64, 2.2M 4481 -> 4683.  (The softmax backward and
        // the cross-entropy gradient have no plan there.)
        if (c.stream && op == kOpSoftmax &&
            (c.G == 128 || (dtype == kBf16 && c.G == 64) || k == kTunedBuckets - 1) &&
            10 * N < 9 * (int64_t)c.P * c.R * c.G)
            return false;
        if (c.stream && c.G > 1 && M <= kFewRows &&
            try_choice(op, dtype, vec, N, Choice{true, 32, 1024, 1}, p))
            return true;
        // A stream workgroup that would be less than half full: the block
        // choice of the bucket below, widened to the row.
        if (c.stream && k > 0 && 2 * N < (int64_t)c.P * c.R) c = kTuned[o][d][k - 1];
        if (try_choice(op, dtype, vec, N, c, p)) {
            exact_groups(op, dtype, vec, N, p);
            return true;
        }
        // a block choice the per-element path does not have: fewer values per lane
        for (Choice b = c; !b.stream && b.P > 8;) {
            b.P /= 2;
            if (try_choice(op, dtype, vec, N, b, p)) return true;
        }
    }
    // Packed bf16 RMSNorm rows past the table: 256 workgroups of 128 values x 512
    // lanes, one on every CU, hold up to 16M elements, at any fill (offset-averaged
    // GB/s, two reads -> on chip: 16777216 elements 3724 -> 5890, 15M 3809 -> 5628,
    // 12M 3927 -> 5256, 9M 4042 -> 4609).
    if (op == kOpRmsnorm && dtype == kBf16 && vec && N > kTunedN[kTunedBuckets - 1])
        return try_choice(op, dtype, vec, N, Choice{true, kPackedP, 512, 256}, p);
    // A configuration the per-element path does not have: the first stream
    // configuration that holds the row with the fewest workgroups.  The per-element
    // path stops at 16 workgroups per row: its longer rows measured no faster on
    // chip than in the two-pass kernel.
    static const int kStreamPR[5][2] = {{64, 512}, {32, 1024}, {64, 256}, {32, 512}, {16, 1024}};
    for (int g = 1; g <= (vec ? 64 : 16); g *= 2)
        for (int j = 0; j < 5; ++j)
            if (try_choice(op, dtype, vec, N, Choice{true, kStreamPR[j][0], kStreamPR[j][1], g}, p))
                return true;
    return false;
}

// Cross-entropy: 16 values per lane for short rows, else 32; as many lanes as the
// row needs, up to 256 lanes (512 for bf16 rows of 32768 or more, which then
// still take two or more steps): 32 KiB of the row per step, which measured best
// for long f32 rows.  bf16 rows of 1025 to 32767 elements take two or more steps
// of the lane count that pads the row least (ties to more lanes, at most eight
// steps, since narrow lane groups reduce more often, and no narrower than keeps
// two 256-lane workgroups per CU of a 256-CU device busy): a row streamed in steps
// overlaps the next step's loads with the reduction of the last, and the lanes
// past the row's end cost about as much as real ones.  Measured on MI355X (GB/s
// averaged over output offsets; "one step": the next power of two above N / 32
// lanes, the choice for f32):
//   N                      1100  1500  2048  3000  4096  5000  6000  8192 12000 20000 24577
//   16384 rows  one step   2439  3310  5461  4079  5905  3702  4366  6162  5200  6017  4625
//               this       2993  4003  5447  5347  6133  5518  5999  6562  6297  6341  5556
//    4096 rows  one step   1613  2099  3731  3067  4589  3046  3640  5071  4562  5329  4104
//               this       1518  2131  3635  3442  5033  4182  4769  5603  5488  5908  4726
static void default_xent(int dtype, int64_t M, int64_t N, int *P, int *R) {
    *P = N <= 512 ? 16 : 32;
    const int64_t rmax = (dtype == kBf16 && N >= 32768) ? 512 : 256;
    int64_t r = next_pow2((N + *P - 1) / *P);
    if (dtype == kBf16 && N > 1024 && N < 32768) {
        int64_t c0 = 16;
        while (c0 < rmax && M * c0 < 2 * 256 * 256) c0 *= 2;
        int64_t best_cap = INT64_MAX;
        for (int64_t c = c0; c <= rmax && c * *P < N; c *= 2) {
            const int64_t step = c * *P, steps = (N + step - 1) / step;
            if (steps <= 8 && steps * step <= best_cap) { best_cap = steps * step; r = c; }
        }
    }
    if (r < 16) r = 16;
    if (r > rmax) r = rmax;
    *R = (int)r;
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// RMSNorm backward: the fastest (P, R, G) measured on MI355X per dtype and N
// bucket (16384 rows, every compiled configuration and 256, 512 or the occupancy
// limit of persistent workgroups timed; one workgroup per CU measured best or
// within a few percent), narrowed to the row as for the forward.
struct BwdChoice {
    int P, R, G;
};
// (the 5120, 8192 and 12288 buckets were added later, where the plans interpolated
// from their neighbours ran up to 23 % slower: bf16 at 5120 elements 3958 -> 4881 GB/s,
// fp32 at 12288 5379 -> 5753; after the split layout changed, bf16 at 32768 and 65536
// took 16 values on 4 and 8 workgroups: 5604 -> 6050 and 5744 -> 6009, offset-averaged)
constexpr int kTunedBwdBuckets = 11;
constexpr int64_t kTunedBwdN[kTunedBwdBuckets] = {256,   1024,  4096,  5120,   8192,  12288,
                                                  16384, 32768, 65536, 131072, 262144};
constexpr bool kBwdAlignedOnly[kTunedBwdBuckets] = {false, false, false, true,  true, true,
                                                    false, false, false, false, false};
static const BwdChoice kTunedRmsBwd[2][kTunedBwdBuckets] = {
    {{8, 32, 1}, {16, 64, 1}, {16, 256, 1}, {32, 256, 1}, {16, 512, 1}, {32, 512, 1},
     {16, 512, 2}, {16, 512, 4}, {32, 512, 4}, {32, 512, 8}, {32, 512, 16}},
    {{16, 16, 1}, {16, 64, 1}, {32, 128, 1}, {8, 1024, 1}, {16, 512, 1}, {32, 512, 1},
     {32, 512, 1}, {16, 512, 4}, {16, 512, 8}, {32, 512, 8}, {32, 512, 16}},
};

static PlanResult plan_rmsnorm_bwd(int dtype, int64_t M, int64_t N, bool vec, Plan *out) {
    const TestOverrides ov = test_overrides();
    const int fP = ov.P, fR = ov.R, fG = ov.G;
    int P, R, G = 1;
    if (fP || fR || fG) {
        P = fP ? fP : 16;
        R = fR ? fR : 512;
        G = fG ? fG : 1;
    } else {
        int k = 0;
        // The 5120, 8192 and 12288 buckets were measured on the 128-bit path; fp32
        // rows on the per-element path keep the plans of the buckets around them.
        // Unaligned bf16 rows, whose loads take no branch, use every bucket and the
        // table's 32 values per lane (16384 rows, GB/s, from 16 values: x2047 3124
        // -> 3582, x4095 3302 -> 3792, x10001 2506 -> 3431, x65537 1519 -> 2480,
        // x131071 2485 -> 3759, x262143 2398 -> 3431).
        while (k < kTunedBwdBuckets - 1 &&
               (kTunedBwdN[k] < N || (!vec && dtype != kBf16 && kBwdAlignedOnly[k])))
            ++k;
        BwdChoice c = kTunedRmsBwd[dtype == kBf16 ? 1 : 0][k];
        if (!vec && c.P > 16 && dtype != kBf16) {  // fp32 per-element: P <= 16, twice the lanes
            c.P = 16;
            if (c.G == 1 && c.R < 512) c.R *= 2; else c.G *= 2;
        }
        P = c.P;
        R = c.R;
        G = c.G;
        if (G == 1) {  // narrowed to the row
            int64_t r = next_pow2((N + P - 1) / P);
            R = (int)(r < 16 ? 16 : (r < R ? r : R));
        } else {
            while (G > 1 && (int64_t)P * R * (G / 2) >= N) G /= 2;
        }
        while ((int64_t)P * R * G < N && G < 32) G *= 2;  // past the table
    }
    if (!rmsbwd_config_ok(dtype, vec, P, R, G)) return kPlanUnsupported;
    if (!vec && R >= 64 && dtype == kBf16 && N < 8) return kPlanUnsupported;
    Plan p;
    p.vec = vec;
    p.stream = true;
    p.P = P;
    p.R = R;
    p.G = G;
    p.max_n = (int64_t)P * R * G;
    if (N > p.max_n) return kPlanUnsupported;
    p.path = G > 1 ? kPathSplit : kPathStream;
    p.block = G == 1 ? block_threads_for(R) : R;
    p.rows_per_block = G == 1 ? rows_per_block_for(R) : 1;
    const int64_t blocks = (M + p.rows_per_block - 1) / p.rows_per_block;
    int64_t parts = kBwdMaxWorkgroups / G;
    if (parts > blocks) parts = blocks;
    if (parts < 1) parts = 1;
    p.max_parts = (int)parts;
    // the exchange area of split rows; with G == 1 the header alone, so that the
    // first word of every workspace is the error word rr_workspace_check reads
    const size_t exch = G > 1 ? align256(grid_ws_bytes(G, parts)) : (size_t)kWsHeader;
    p.part_off = exch;
    p.ws_bytes = p.part_off + align256((size_t)parts * (size_t)N * 4u);
    *out = p;
    return kPlanOk;
}

PlanResult make_plan(int op, int dtype, int64_t M, int64_t N, bool vec, Plan *out) {
    if (!out) return kPlanInvalid;
    if (op == kOpRmsnormBwd) {
        if ((dtype != kF32 && dtype != kBf16) || M < 0 || N < 1 || N > INT32_MAX) return kPlanInvalid;
        return plan_rmsnorm_bwd(dtype, M, N, vec, out);
    }
    if ((op != kOpSoftmax && op != kOpRmsnorm && op != kOpXent && op != kOpXentGrad &&
         op != kOpSoftmaxBwd) ||
        (dtype != kF32 && dtype != kBf16) || M < 0 || (M > 0 && N < 1))
        return kPlanInvalid;
    if (op == kOpXentGrad && N > INT32_MAX) return kPlanInvalid;
    if (N < 1) N = 1;  // M == 0: any plan will do, nothing is launched
    Plan p;
    p.vec = vec;
    const TestOverrides ov = test_overrides();
    const int fP = ov.P, fR = ov.R, fG = ov.G;

    if (op == kOpXent) {
        if (N > INT32_MAX) return kPlanInvalid;
        int P, R;
        default_xent(dtype, M, N, &P, &R);
        if (fP) P = fP;
        if (fR) R = fR;
        if (!xent_config_exists(P, R)) return kPlanUnsupported;
        p.path = kPathXent;
        p.P = P;
        p.R = R;
        p.G = 1;
        p.max_n = INT32_MAX;
        p.ws_bytes = 0;
        fill_geometry(&p);
        *out = p;
        return kPlanOk;
    }

    const bool force_stream = ov.kind == kForceStream;
    const bool force_block = ov.kind == kForceBlock;
    const bool force_long = ov.kind == kForceLong;
    const bool long_op =
        op == kOpSoftmax || op == kOpRmsnorm || op == kOpSoftmaxBwd || op == kOpXentGrad;
    if (long_op && (force_long || (!fP && !fR && !fG && !force_stream && !force_block &&
                                   !default_row(op, dtype, vec, M, N, &p)))) {
        // past every on-chip plan: read the row twice
        if (N > kLongMaxN) return kPlanUnsupported;
        if (!vec && dtype == kBf16 && N < 8) return kPlanUnsupported;  // see below
        p = Plan{};
        p.vec = vec;
        p.stream = true;
        p.path = kPathLong;
        p.P = vec ? kLongP : kLongPElem;
        p.R = kLongR;
        // the softmax backward reads two rows (y and dy) per pass
        p.G = long_row_groups((op == kOpSoftmaxBwd ? 2 : 1) * N * (dtype == kBf16 ? 2 : 4));
        p.max_n = kLongMaxN;
        p.ws_bytes = grid_ws_bytes(p.G, M);
        p.block = kLongR;
        p.rows_per_block = 1;
        *out = p;
        return kPlanOk;
    }
    if (fP || fR || fG || force_stream || force_block) {
        p.stream = force_stream || (!force_block && fG > 1);
        p.P = fP ? fP : (p.stream ? 64 : 16);
        p.R = fR ? fR : (p.stream ? 512 : 256);
        p.G = fG ? fG : 1;
        const bool ok = p.stream ? stream_config_ok(op, dtype, vec, p.P, p.R, p.G)
                                 : (p.G == 1 && block_config_ok(op, dtype, vec, p.P, p.R));
        if (!ok) return kPlanUnsupported;
    } else if (!default_row(op, dtype, vec, M, N, &p)) {
        return kPlanUnsupported;
    }
    const int P = p.P, R = p.R, G = p.G;
    p.max_n = (int64_t)P * R * G;
    if (N > p.max_n) return kPlanUnsupported;
    // Unaligned bf16 rows shorter than 16 bytes are read element by element, which
    // only lane groups of fewer than 64 lanes compile.
    if (!vec && R >= 64 && dtype == kBf16 && N < 8) return kPlanUnsupported;
    p.path = !p.stream ? kPathRow : (G > 1 ? kPathSplit : kPathStream);
    p.ws_bytes = G > 1 ? grid_ws_bytes(G, M) : 0;
    if (p.stream) {
        p.block = R;
        p.rows_per_block = 1;
    } else {
        fill_geometry(&p);
    }
    *out = p;
    return kPlanOk;
}

}  // namespace rr
