// Skip-Softmax (BLASST) FlashAttention forward for AMD Instinct MI355X (gfx950).
//
// The method: "Skip-Softmax" design document of vLLM-Omni, section
// "Algorithm"; "Skip-Softmax" page of the vLLM-Omni documentation, sections
// "The online-softmax pass" and "The skip test".  The C ABI is declared in
// include/ssa.h.
//
// Work decomposition.  One workgroup = 8 waves = 256 query rows of one
// (sequence, head); each wave owns 32 rows, and the two waves 2g, 2g+1 form
// the 64-row vote group g of the skip test.  Workgroups are renumbered so
// that each XCD works through whole heads, sharing K/V tiles in its L2; in a
// packed batch each XCD takes an eighth of every sequence's work.
// Key tiles of 128 keys stream through LDS (K and V double buffered, shared
// by all eight waves), copied from global memory straight into LDS by
// buffer loads with the LDS-destination bit; keys past the end of the
// sequence lie outside the buffer resource's range and arrive as zeros.
//
// Ping-pong schedule.  Two waves share each SIMD: waves 0-3 (group A) and
// 4-7 (group B).  Each tile goes through two phases per wave, one per slot,
// with a workgroup barrier ending every slot:
//   MFMA phase     O^T += V^T P^T of the previous tile (if it was kept), then
//                  the scores S^T = K Q^T of this tile
//   softmax phase  row maximum, the vote group's skip decision, and for a
//                  kept tile the online-softmax update with P in bf16
// Group B runs one slot behind group A, so in every slot one wave of each
// SIMD feeds the matrix cores while the other runs the softmax.  A call
// without the skip test (lambda = 0) runs a separate instance of the kernel
// without the vote, whose group A issues the V copies inside its QK^T steps
// (group B still issues the K copies, after its softmax phase).
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, fp32 accumulate).  S^T is
// 4 key blocks of 32 x 32: a lane holds one query row and 16 keys per block,
// so row reductions are in-lane plus one exchange between the wave halves.
// The K operand's rows are permuted so that accumulator registers 8t..8t+7
// hold 8 consecutive keys; rounded to bf16 they are directly the B operand
// (P^T) of O^T = V^T P^T, whose A operand V^T comes from the natural-layout
// V tile through LDS transpose reads (ds_read_b64_tr_b16).
//
// The skip test runs on fp32 scores in log space before any exponential:
// tile_max[i] - m[i] < ln(lambda) for every valid row of the vote group,
// m the true running maximum over the kept tiles.  A skipped tile costs only
// its QK^T and row maximum; m, l and O are left untouched.
//
// Virtual tiles (the compensated entry).  Each vote group records its skip
// decisions; after the last tile, every skipped tile t adds one virtual key,
// the mean of its keys with score + ln(n_t), and the mean of its values to
// the row's softmax ("Triage: Skip, Skim, or Refine Attention Tiles in Video
// Diffusion Transformers", section 6.1).  The tile means come from a
// pre-pass; the virtual scores and their P.V run on MFMA, 32 tiles at a time.
// They never enter the running maximum the skip test uses.
//
// Exponent reference.  The exponentials use a per-row reference r <= m and
// O, l are rescaled only when m climbs more than kRescaleLog2 binades above
// r (then r = m).  This changes only rounding: O / l and r + ln(l) do not
// depend on the reference, and P = exp(s - r) stays below 2^kRescaleLog2.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <type_traits>

#include "ssa.h"

// Workspace of ssa_fwd_virtual_noalloc (the per-tile mean keys and values),
// for callers that cannot allocate: one array per GPU, held until the
// process ends.  Host code never passes this name to a kernel or a copy (on
// the host it is only a stand-in for the symbol): it uses the device address
// that hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = SSA_VIRTUAL_NOALLOC_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kD = 128;
constexpr int kBQ = 64;                 // rows per vote group
constexpr int kBK = 128;                // keys per tile
constexpr int kRowsPerWave = 32;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWG = kRowsPerWave * kWaves;
constexpr int kRowBytes = kD * 2;                  // one bf16 row of 128 channels
constexpr int kTileBytes = kBK * kRowBytes;        // 32 KB
constexpr int kCopyPerWave = kTileBytes / (kWaves * 1024);   // 1 KB DMA instructions per wave per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleLog2 = 16.f;               // P <= 2^16 before a rescale is forced
constexpr int kSpinLimit = 1 << 14;                 // default polls of the partner's vote before giving up
constexpr int kMaxSpinLimit = 1 << 24;
constexpr unsigned kRsrcWord3 = 0x00020000u;       // raw buffer, 32-bit data format
constexpr int kXcds = 8;                            // XCDs of an MI355X, each with its own L2
constexpr int kCompWords = 64;                      // virtual tiles: 32 skip bits per word, up to 2048 tiles
constexpr int kCompRound = 128;                     // virtual tiles staged in LDS per round
constexpr int kRow8 = kD;                           // one FP8 row of 128 channels (bytes)
constexpr int kTile8Bytes = kBK * kRow8;            // 16 KB
constexpr int kMaxTilesFp8 = 4096;                  // FP8 scores: K tile scales staged in LDS

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) int i32x8;
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  float* maxp;                 // largest softmax weight of each row (nullable)
  int32_t* counts;
  uint8_t* mask;
  float* margin;
  const int32_t* cu_seqlens;   // null: fixed-length [B, H, S, D]
  const uint16_t* kbar;        // virtual tiles: [B, H, nKT, 2, D] bf16 mean key (hi, lo)
  const uint16_t* vbar;        // virtual tiles: [B, H, nKT, D] bf16 mean value
  const uint8_t* q8;           // FP8 scores: E4M3 codes [B, H, S, D] of q and k
  const uint8_t* k8;
  const float* q_scale;        // FP8 scores: [B, H, S] per-token scale of q
  const float* k_scale;        // FP8 scores: [B, H, nKT] per-tile scale of k
  int nseq;                    // B
  int H;
  int S;                       // fixed length, or max_seqlen
  int qgroups;                 // workgroups per (sequence, head)
  long long tok_stride;        // elements between consecutive tokens
  long long head_stride;       // elements between heads
  long long seq_stride;        // elements between batch entries (fixed length)
  float scale;
  float scale_log2e;
  float ln_lambda;             // used when lambda_per_seq == 0
  int vote;                    // 0: lambda == 0, nothing is skipped
  int lambda_per_seq;          // 1: ln(lambda_b) = ln(factor / S_b)
  int spin_limit;              // debug instance: polls of the partner's half of the vote before the tile is kept
  double factor;
};

// XOR swizzle of the 16-byte chunk index within a 256-byte LDS row, a linear
// map of the row's low 4 bits.  It makes the 16-byte K operand reads (rows
// permuted by key_perm) and the transpose reads of V hit distinct banks for
// every group of 8 and of 16 lanes; whole-row writes are unaffected.
__device__ __forceinline__ int swz(int r) {
  return ((r & 1) ? 4 : 0) ^ ((r & 2) ? 10 : 0) ^ ((r & 4) ? 1 : 0) ^ ((r & 8) ? 3 : 0);
}

// Key row that MFMA row m (0..31) of a 32-key block loads.  With this
// permutation accumulator register r of lane half hf holds key
// 16 * (r / 8) + 8 * hf + (r % 8) of the block.
__device__ __forceinline__ int key_perm(int m) {
  const int a = m >> 3, hh = (m >> 2) & 1, j = m & 3;
  return 16 * (a >> 1) + 8 * hh + 4 * (a & 1) + j;
}

// Both halves of the wave receive f(x[lane], x[lane ^ 32]).
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The vote's arithmetic, rounded step by step (never fused into an FMA):
// tile_max = fl(raw_max * scale), margin = fl(tile_max - m).  Every entry
// point then takes bit-identical decisions.
__device__ __forceinline__ float scaled_max(float raw_max, float scale) {
#pragma clang fp contract(off)
  return raw_max * scale;
}
__device__ __forceinline__ float vote_margin(float tile_max, float m) {
#pragma clang fp contract(off)
  return tile_max - m;
}

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Two floats to two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, (int)kRsrcWord3);
}

// Packed batches: the length of sequence sb as the work map counts it (0
// for a length that is negative or above max_seqlen, and past the last
// sequence).
__device__ __forceinline__ int varlen_len(const Params& p, int sb) {
  int len = sb < p.nseq ? p.cu_seqlens[sb + 1] - p.cu_seqlens[sb] : 0;
  return (len < 0 || len > p.S) ? 0 : len;
}

// Inclusive prefix sum over the 64 lanes of the wave.
__device__ __forceinline__ int wave_incl_sum(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// Query blocks (of 64 rows) of the sequences before sequence b, and of all
// sequences: the offset and row length of the skip-count layout
// [H, sum_b ceil(S_b / 64)].
__device__ __forceinline__ void varlen_qblocks(const Params& p, int b, int lane, long long& off, long long& total) {
  off = 0;
  total = 0;
  for (int base0 = 0; base0 < p.nseq; base0 += 64) {
    const int nqb = (varlen_len(p, base0 + lane) + kBQ - 1) / kBQ;
    const int incl = wave_incl_sum(nqb, lane);
    if (b >= base0 && b < base0 + 64)
      off = total + __builtin_amdgcn_readlane(incl, b - base0) - __builtin_amdgcn_readlane(nqb, b - base0);
    total += __builtin_amdgcn_readlane(incl, 63);
  }
}

// kDense: the lambda = 0 instance (no vote); it differs from the general one
// only in when and by which wave the K/V copies are issued.
template <bool kDebug, bool kComp, bool kFp8, bool kDense>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ssa_fwd_kernel(const Params p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k[2][kFp8 ? kTile8Bytes : kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v[2][kTileBytes];
  __shared__ int vote_lds[kWaves];      // (tile << 1) | pass of the wave's half of the vote
  __shared__ int vote_timeout[kWaves / 2];   // 1: a wave of the vote group gave up waiting for its partner
  __shared__ float margin_lds[kWaves];  // debug: the wave's margin for the tile
  __shared__ uint32_t comp_bits[kComp ? kWaves / 2 * kCompWords : 1];   // skip bits per vote group
  __shared__ float kscale_lds[kFp8 ? kMaxTilesFp8 : 1];                 // FP8 scores: scale of each K tile

  // XCD-aware work order.  The dispatcher hands workgroup L (linear id) to
  // XCD L % 8, each XCD with its own L2.  Renumber so that XCD x runs one
  // contiguous range of the (query group, head, sequence) list: the 32 CUs
  // of an XCD then stream the same head's K/V tiles at the same time and
  // share them in their L2, instead of two heads per XCD at half the reuse.
  // Within a head the query groups run last to first: keys are visited in
  // ascending order, so early queries tend to meet their largest scores
  // early and skip more tiles, and dispatching the costlier late groups
  // first leaves the cheap ones to fill the end of the launch.
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, hf = lane >> 5;
  const bool group_b = wave >= 4;
  int qg, h, b;
  long long tok0 = 0;
  int S_b = p.S;
  if (p.cu_seqlens == nullptr) {
    const int gx = gridDim.x, gy = gridDim.y;
    const int n = gx * gy * (int)gridDim.z;
    const int L = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
    const int per = n / kXcds, rem = n % kXcds, xcd = L % kXcds;
    const int W = xcd * per + (xcd < rem ? xcd : rem) + L / kXcds;
    qg = gx - 1 - W % gx;
    h = (W / gx) % gy;
    b = W / (gx * gy);
  } else {
    // Packed batch: sequences differ in length, so equal ranges of a grid
    // padded to max_seqlen would hand some XCDs all the long sequences.
    // Sequence b has I_b = H * ceil(S_b / 256) work items in (head, query
    // group) order; XCD x takes the x-th of eight near-equal contiguous
    // chunks of every sequence's items, sequences in order, so each XCD gets
    // an eighth of every sequence (and still whole runs of one head).  The
    // 1-D grid holds 8 * nseq * ceil(H * ceil(max_seqlen / 256) / 8)
    // workgroups; those past the end of their XCD's list return at once.
    // One wave-wide prefix scan per 64 sequences finds this workgroup's
    // sequence.  Sequences whose length is negative or above max_seqlen get
    // no items.
    const int L = blockIdx.x;
    const int xcd = L % kXcds;
    int r = L / kXcds;
    b = -1;
    int local = 0;
    for (int base0 = 0; base0 < p.nseq && b < 0; base0 += 64) {
      const long long items = (long long)p.H * ((varlen_len(p, base0 + lane) + kRowsPerWG - 1) / kRowsPerWG);
      const int cnt = (int)(items * (xcd + 1) / kXcds - items * xcd / kXcds);
      const int incl = wave_incl_sum(cnt, lane);
      const int total = __builtin_amdgcn_readlane(incl, 63);
      if (r < total) {
        const int ln = __builtin_ctzll(__builtin_amdgcn_ballot_w64(incl > r));   // first lane past r
        b = base0 + ln;
        local = r - (__builtin_amdgcn_readlane(incl, ln) - __builtin_amdgcn_readlane(cnt, ln));
      } else {
        r -= total;
      }
    }
    if (b < 0) return;   // nothing left in this XCD's list
    tok0 = p.cu_seqlens[b];
    S_b = p.cu_seqlens[b + 1] - (int)tok0;
    const int nqg = (S_b + kRowsPerWG - 1) / kRowsPerWG;
    const int item = (int)((long long)p.H * nqg * xcd / kXcds) + local;
    h = item / nqg;
    qg = nqg - 1 - item % nqg;   // last query group first, as above
  }
  if (qg * kRowsPerWG >= S_b) return;   // whole workgroup past the end of its sequence

  const long long base = (p.cu_seqlens != nullptr ? tok0 * p.tok_stride : (long long)b * p.seq_stride) +
                         (long long)h * p.head_stride;
  const uint32_t ts_bytes = (uint32_t)(p.tok_stride * 2);
  // Byte range of this (sequence, head): its last token's row ends the range.
  const uint32_t range = (uint32_t)((long long)(S_b - 1) * p.tok_stride * 2 + kRowBytes);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + base, range);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + base, range);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + base, range);

  float ln_lambda = p.ln_lambda;
  if (p.lambda_per_seq) ln_lambda = (float)log(p.factor / (double)S_b);
  const bool vote = !kDense && p.vote != 0;

  const int nkt = (S_b + kBK - 1) / kBK;
  const int wrow0 = qg * kRowsPerWG + wave * kRowsPerWave;   // this wave's first row
  const int qb = (qg * kRowsPerWG) / kBQ + (wave >> 1);      // vote group (64-row q-block)
  const bool valid = wrow0 + c < S_b;

  // Q^T operand fragments: qf[s] = Q[wrow0 + c][16 s + 8 hf .. +7] (rows past
  // the end read as zeros).
  bf16x8 qf[8];
  // FP8 scores: Q^T operand of the 32 x 32 x 64 MFMA, qf8[s] = codes
  // Q8[wrow0 + c][64 s + 32 hf .. +31]; K tiles are E4M3 codes as well, and
  // the scores are scale * q_scale[row] * k_scale[tile] * (Q8 . K8).
  i32x8 qf8[2];
  float sq_row = 0.f;                     // scale * q_scale of this lane's row
  const long long head8 = ((long long)b * p.H + h) * p.S;   // first token of this head (FP8 arrays)
  __amdgpu_buffer_rsrc_t rk8 = rk;
  if constexpr (kFp8) {
    const uint32_t range8 = (uint32_t)S_b * kRow8;
    const __amdgpu_buffer_rsrc_t rq8 = make_rsrc(p.q8 + head8 * kRow8, range8);
    rk8 = make_rsrc(p.k8 + head8 * kRow8, range8);
    const uint32_t off = (uint32_t)(wrow0 + c) * kRow8 + 32u * hf;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq8, off + 64u * s, 0, 0));
      const u32x4 hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq8, off + 64u * s + 16u, 0, 0));
      qf8[s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    // padding rows take any positive factor: they neither vote nor are stored
    sq_row = valid ? p.scale * p.q_scale[head8 + wrow0 + c] : p.scale;
    // the head's K tile scales, read by every softmax phase
    for (int t = tid; t < nkt; t += kThreads) kscale_lds[t] = p.k_scale[((long long)b * p.H + h) * nkt + t];
  } else {
    const uint32_t off = (uint32_t)(wrow0 + c) * ts_bytes + 16u * hf;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qf[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off + 32u * s, 0, 0));
  }

  // ---- tile copy: global -> LDS, 16 bytes per lane per instruction ----
  // Instruction j of a 16-row block fills its rows 4 j .. 4 j + 3 (1 KB);
  // lane l lands at byte 16 l: row + l / 16, physical chunk l % 16, which
  // holds logical chunk (l % 16) ^ swz(row).  Rows 16 apart share a swizzle,
  // so the blocks of a wave differ by uniform offsets.
  uint32_t copy_off[kCopyPerWave];
#pragma unroll
  for (int j = 0; j < kCopyPerWave; ++j) {
    const int r = 4 * j + (lane >> 4);
    copy_off[j] = (uint32_t)r * ts_bytes + 16u * (uint32_t)((lane & 15) ^ swz(r));
  }
  // The 16-row block `blk` (0..7) of tile kt into the LDS tile at dst.
  auto copy_block = [&](const __amdgpu_buffer_rsrc_t& rs, int kt, unsigned char* dst, int blk) __attribute__((always_inline)) {
    const uint32_t goff = (uint32_t)(kt * kBK + 16 * blk) * ts_bytes;
#pragma unroll
    for (int j = 0; j < kCopyPerWave; ++j)
      // The whole offset goes in the per-lane (range-checked) voffset.
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_PTR(void, dst + (16 * blk + 4 * j) * kRowBytes), 16,
                                               copy_off[j] + goff, 0, 0, 0);
  };

  // FP8 K tile copy: 128-byte rows, 8 rows (1 KB) per instruction; lane l
  // lands at row + l / 8, physical chunk l % 8, which holds logical chunk
  // (l % 8) ^ swz8(row) with swz8(row) = (row / 2) % 8 (equal for rows 16
  // apart).
  uint32_t copy_off8[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 8 * j + (lane >> 3);
    copy_off8[j] = (uint32_t)r * kRow8 + 16u * (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
  }
  // The 16-row block `blk` (0..7) of FP8 K tile kt into the LDS tile at dst.
  auto copy_block8 = [&](int kt, unsigned char* dst, int blk) __attribute__((always_inline)) {
    const uint32_t goff = (uint32_t)(kt * kBK + 16 * blk) * kRow8;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk8, LDS_PTR(void, dst + (16 * blk + 8 * j) * kRow8), 16,
                                               copy_off8[j] + goff, 0, 0, 0);
  };
  auto copy_k = [&](int kt, unsigned char* dst, int blk) __attribute__((always_inline)) {
    if constexpr (kFp8) copy_block8(kt, dst, blk);
    else copy_block(rk, kt, dst, blk);
  };
  // The in-loop copies: instruction j of block blk of tile kt (of V when
  // is_v, else of bf16 K) into the LDS tile at byte offset lds_tile, as in
  // copy_block but through inline assembly.  The compiler does not see these
  // loads, so it never makes an LDS read of the other buffer wait for them;
  // the vmcnt(0) at the end of every odd slot is their only wait.
  const uint32_t lds_k_off = (uint32_t)(uintptr_t)LDS_PTR(unsigned char, &lds_k[0][0]);
  const uint32_t lds_v_off = (uint32_t)(uintptr_t)LDS_PTR(unsigned char, &lds_v[0][0]);
  auto copy_one_untracked = [&](bool is_v, int kt, uint32_t lds_tile, int blk, int j) __attribute__((always_inline)) {
    const uint32_t goff = (uint32_t)(kt * kBK + 16 * blk) * ts_bytes;
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_tile + (uint32_t)((16 * blk + 4 * j) * kRowBytes));
    if (is_v)
      asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" :: "v"(copy_off[j] + goff), "s"(rv), "{m0}"(m0));
    else
      asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" :: "v"(copy_off[j] + goff), "s"(rk), "{m0}"(m0));
  };
  // The same for instruction j (0 or 1) of block blk of FP8 K tile kt.
  auto copy_one_untracked8 = [&](int kt, uint32_t lds_tile, int blk, int j) __attribute__((always_inline)) {
    const uint32_t goff = (uint32_t)(kt * kBK + 16 * blk) * kRow8;
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_tile + (uint32_t)((16 * blk + 8 * j) * kRow8));
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" :: "v"(copy_off8[j] + goff), "s"(rk8), "{m0}"(m0));
  };

  // Per-lane LDS byte offsets of the operand reads.
  // K operand (A of S^T): row 32 kb + key_perm(c), logical chunk 2 s + hf.
  const int krow = key_perm(c);
  const int kswz = swz(krow);
  const int kswz8 = (krow >> 1) & 7;     // FP8 K rows: swz8 of row 32 kb + krow
  // V^T operand (A of O^T) via transpose reads: within 16-lane group g the
  // lane 4 e + q supplies row 8 hf + 4 ih + e (plus the 16-key step base),
  // channels 32 db + 16 (g % 2) + 4 q .. +3.
  int voff[2][4];
  {
    const int ve = (lane & 15) >> 2, vq = lane & 3, vg = (lane >> 4) & 1;
#pragma unroll
    for (int ih = 0; ih < 2; ++ih) {
      const int row = 8 * hf + 4 * ih + ve;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int lc = 4 * db + 2 * vg + (vq >> 1);
        voff[ih][db] = row * kRowBytes + 16 * (lc ^ swz(row)) + 8 * (vq & 1);
      }
    }
  }

  float m_run = -INFINITY;    // running max (natural units), drives the vote
  float mb_ref = -INFINITY;   // exponent reference, log2 units
  float l = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  int nskip = 0;
  bool timed_out = false;   // this wave gave up waiting for its partner's half of a vote
  uint32_t comp_cur = 0;   // virtual tiles: skip bits of the current 32-tile word

  // Scores of the tile between its MFMA and softmax phases.  The softmax
  // phase of a kept tile overwrites them in place with P in bf16: register
  // 4 t2 + w of block kb holds the pair of keys 8 t2 + 2 w, + 1, and
  // registers 4 t2 .. 4 t2 + 3 are the B operand (P^T) of P.V step (kb, t2).
  f32x16 sacc[4];
  bool p_ready = false;

  // ---- MFMA phase: O^T += V^T P^T for the previous tile (if kept), then
  // S^T = K Q^T for tile kt.  One stream of up to 64 MFMAs whose A operands
  // (V^T by transpose reads, then K) come from LDS through one ring of
  // fragments read kRing steps ahead; four independent accumulators in each
  // half hide the MFMA latency.  With cp_c set (the dense instance, group A)
  // the QK^T steps also issue the copy of V(kt), one instruction every fourth
  // MFMA, into the V buffer this phase does not read.
  constexpr int kRing = 8;
  auto mfma_phase = [&](auto pv_c, auto qk_c, auto cp_c, int kt) __attribute__((always_inline)) {
    constexpr bool kPV = decltype(pv_c)::value, kQK = decltype(qk_c)::value, kCopy = decltype(cp_c)::value;
    constexpr int n0 = kPV ? 0 : 32, n1 = kQK ? 64 : 32;   // steps [n0, n1): < 32 P.V, >= 32 QK^T
    const unsigned char* vl = lds_v[(kt - 1) & 1];
    const unsigned char* kl = lds_k[kt & 1];
    auto frag = [&](int i) __attribute__((always_inline)) {
      if (i < 32) {
        const int kb = i >> 3, t2 = (i >> 2) & 1, db = i & 3;
        const unsigned char* vstep = vl + (32 * kb + 16 * t2) * kRowBytes;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vstep + voff[0][db]));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vstep + voff[1][db]));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        const u32x4 av = {l2[0], l2[1], h2[0], h2[1]};
        return __builtin_bit_cast(bf16x8, av);
      }
      const int s = (i - 32) >> 2, kb = i & 3;
      const int off = kb * 32 * kRowBytes + krow * kRowBytes + 16 * ((2 * s + hf) ^ kswz);
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kl + off));
    };
    bf16x8 ring[kRing];
#pragma unroll
    for (int i = 0; i < kRing; ++i) ring[i] = frag(n0 + i);
#pragma unroll
    for (int i = n0; i < n1; ++i) {
      const bf16x8 a = ring[(i - n0) % kRing];
      if (i + kRing < n1) ring[(i - n0) % kRing] = frag(i + kRing);
      if (i < 32) {
        const int kb = i >> 3, t2 = (i >> 2) & 1, db = i & 3;
        const u32x4 pb = {__float_as_uint(sacc[kb][4 * t2]), __float_as_uint(sacc[kb][4 * t2 + 1]),
                          __float_as_uint(sacc[kb][4 * t2 + 2]), __float_as_uint(sacc[kb][4 * t2 + 3])};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pb), oacc[db], 0, 0, 0);
      } else {
        const int s = (i - 32) >> 2, kb = i & 3;
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], s == 0 ? f32x16{} : sacc[kb], 0, 0, 0);
      }
      if constexpr (kCopy) {
        // the wave's blocks 2 wave and 2 wave + 1 of V(kt)
        if (i >= 32 && (i - 32) % 4 == 0) {
          const int cj = (i - 32) / 4;
          copy_one_untracked(true, kt, lds_v_off + (uint32_t)((kt & 1) * kTileBytes), 2 * wave + cj / kCopyPerWave,
                             cj % kCopyPerWave);
        }
      }
    }
    // Keep the order: reads for step i + kRing go out right after MFMA i.
    __builtin_amdgcn_sched_group_barrier(0x100, (kPV ? 2 : 1) * kRing, 0);
#pragma unroll
    for (int i = n0; i < n1; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + kRing < n1) {
        if (i + kRing < 32)
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        else
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  };

  // ---- FP8-score MFMA phase: O^T += V^T P^T for the previous tile (bf16,
  // as above), then S^T = K8 Q8^T for tile kt with 8 MFMAs of 32 x 32 x 64
  // (E4M3 x E4M3, fp32 accumulate).  One ring of 8 slots of 16 bytes feeds
  // both: a V^T fragment takes one slot (two transpose reads), a K fragment
  // two (two 16-byte reads); slots are refilled 8 loads ahead.
  auto mfma_phase8 = [&](auto pv_c, auto qk_c, int kt) __attribute__((always_inline)) {
    constexpr bool kPV = decltype(pv_c)::value, kQK = decltype(qk_c)::value;
    constexpr int L0 = kPV ? 0 : 32, L1 = kQK ? 48 : 32;   // loads [L0, L1): < 32 V^T, >= 32 K halves
    const unsigned char* vl = lds_v[(kt - 1) & 1];
    const unsigned char* kl = lds_k[kt & 1];
    auto load = [&](int L) __attribute__((always_inline)) {
      if (L < 32) {
        const int kb = L >> 3, t2 = (L >> 2) & 1, db = L & 3;
        const unsigned char* vstep = vl + (32 * kb + 16 * t2) * kRowBytes;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vstep + voff[0][db]));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vstep + voff[1][db]));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
      }
      const int j = (L - 32) >> 1, hh = (L - 32) & 1;
      const int s = j >> 2, kb = j & 3;
      const int off = (32 * kb + krow) * kRow8 + 16 * ((4 * s + 2 * hf + hh) ^ kswz8);
      return *reinterpret_cast<const u32x4*>(kl + off);
    };
    u32x4 ring[kRing];
#pragma unroll
    for (int i = 0; i < kRing; ++i) ring[i] = load(L0 + i);
    if constexpr (kPV) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const u32x4 a = ring[i % kRing];
        if (i + kRing < L1) ring[i % kRing] = load(i + kRing);
        const int kb = i >> 3, t2 = (i >> 2) & 1, db = i & 3;
        const u32x4 pb = {__float_as_uint(sacc[kb][4 * t2]), __float_as_uint(sacc[kb][4 * t2 + 1]),
                          __float_as_uint(sacc[kb][4 * t2 + 2]), __float_as_uint(sacc[kb][4 * t2 + 3])};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, pb),
                                                           oacc[db], 0, 0, 0);
      }
    }
    if constexpr (kQK) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int La = 32 + 2 * j;
        const u32x4 a0 = ring[La % kRing], a1 = ring[(La + 1) % kRing];
        if (La + kRing < L1) ring[La % kRing] = load(La + kRing);
        if (La + 1 + kRing < L1) ring[(La + 1) % kRing] = load(La + 1 + kRing);
        const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        const int s = j >> 2, kb = j & 3;
        // zero scale operands select the unscaled E4M3 x E4M3 instruction
        sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf8[s], s == 0 ? f32x16{} : sacc[kb], 0, 0, 0,
                                                                   0, 0, 0);
      }
    }
    // Keep the order: the refills for a slot go out right after the MFMA
    // that consumed it.
    __builtin_amdgcn_sched_group_barrier(0x100, kPV ? 2 * kRing : kRing, 0);
    if constexpr (kPV) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + kRing < 32)
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        else if (i + kRing < L1)
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    if constexpr (kQK) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (32 + 2 * j + 1 + kRing < L1) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
  };

  // ---- softmax phase of tile kt: row maximum, this wave's half of the
  // vote, the vote group's decision (the partner wave runs the same phase in
  // the same slot and publishes through LDS), and for a kept tile the
  // online-softmax update with P = exp(s - r) packed to bf16.
  auto softmax_phase = [&](int kt) __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, sacc[kb][r]);
    if ((kt + 1) * kBK > S_b) {
      // Keys past the end of the sequence score -inf; redo the maximum.
      mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * kBK + 32 * kb + 16 * (r >> 3) + 8 * hf + (r & 7);
          if (key >= S_b) sacc[kb][r] = -INFINITY;
          mx = __builtin_elementwise_maximum(mx, sacc[kb][r]);
        }
    }
    // Factor from accumulator units to scores (one product per row and tile
    // for FP8 scores, rounded once; the vote uses it exactly as below).
    float sfac = p.scale, sfac_log2e = p.scale_log2e;
    if constexpr (kFp8) {
      sfac = sq_row * kscale_lds[kt];
      sfac_log2e = sfac * kLog2e;
    }
    const float tmax = scaled_max(halves_max(mx), sfac);
    const float dmargin = vote_margin(tmax, m_run);
    bool skip = false;
    if (vote || kDebug) {
      const bool own_pass = __builtin_amdgcn_ballot_w64(valid && !(dmargin < ln_lambda)) == 0;
      if constexpr (kDebug) {
        float md = valid ? dmargin : -INFINITY;
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) md = fmaxf(md, __shfl_xor(md, off));
        if (lane == 0) margin_lds[wave] = md;
      }
      // The vote carries the tile index, so no reset is needed between tiles;
      // the debug margin is published before it (release / acquire).
      constexpr int kPub = kDebug ? __ATOMIC_RELEASE : __ATOMIC_RELAXED;
      constexpr int kSub = kDebug ? __ATOMIC_ACQUIRE : __ATOMIC_RELAXED;
      if (lane == 0)
        __hip_atomic_store(&vote_lds[wave], (kt << 1) | (own_pass ? 1 : 0), kPub, __HIP_MEMORY_SCOPE_WORKGROUP);
      // The partner publishes in this same slot; the bound only guards
      // against a wave that never arrives.  Each poll is one LDS round trip;
      // sleeping between polls measured slightly slower.  A wave that gives
      // up keeps the tile (always exact) and flags its vote group, whose
      // skip count is then stored as -1 - count.  The debug instance takes
      // the bound from the host, so that a test can drive this path; the
      // product instances keep it a constant (a per-tile flag store, or a
      // loop bound read from the arguments, measured several percent slower
      // in skip mode).
      int pv = 0;
      bool got = false;
      const int spin_limit = kDebug ? p.spin_limit : kSpinLimit;
      for (int spin = 0; spin < spin_limit; ++spin) {
        pv = __hip_atomic_load(&vote_lds[wave ^ 1], kSub, __HIP_MEMORY_SCOPE_WORKGROUP);
        if ((pv >> 1) == kt) {
          got = true;
          break;
        }
      }
      timed_out |= !got;
      skip = vote && own_pass && got && (pv & 1) != 0;
      if constexpr (kDebug) {
        if (lane == 0 && (wave & 1) == 0) {
          const long long nqb = (S_b + kBQ - 1) / kBQ;
          if (qb < nqb) {
            const long long idx = (((long long)b * p.H + h) * nqb + qb) * nkt + kt;
            if (p.mask != nullptr) p.mask[idx] = skip ? 1 : 0;
            if (p.margin != nullptr) p.margin[idx] = fmaxf(margin_lds[wave], margin_lds[wave + 1]);
          }
        }
      }
    }
    if constexpr (kComp) {
      // The decision is uniform over the wave; the even wave of the group
      // stores each completed word of 32 decisions.
      if (skip) comp_cur |= 1u << (kt & 31);
      if ((kt & 31) == 31 || kt == nkt - 1) {
        if (lane == 0 && (wave & 1) == 0) comp_bits[(wave >> 1) * kCompWords + (kt >> 5)] = comp_cur;
        comp_cur = 0;
      }
    }
    if (skip) {
      ++nskip;
      p_ready = false;
      return;
    }
    m_run = fmaxf(m_run, tmax);
    if (__builtin_amdgcn_ballot_w64(m_run * kLog2e > mb_ref + kRescaleLog2) != 0) {
      const float nb = m_run * kLog2e;
      const float alpha = __builtin_amdgcn_exp2f(mb_ref - nb);   // 0 on the first kept tile
      mb_ref = nb;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int r = 8 * t2 + 2 * w;
          const float e0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], sfac_log2e, -mb_ref));
          const float e1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r + 1], sfac_log2e, -mb_ref));
          rs += e0 + e1;
          sacc[kb][4 * t2 + w] = __uint_as_float(pack_bf16(e0, e1));
        }
    l += rs;
    p_ready = true;
  };

  // ---- main loop over slots; each slot ends with a workgroup barrier ----
  // Group A runs the MFMA phase of tile slot / 2 on even slots and its
  // softmax phase on odd slots; group B runs what A ran one slot earlier.
  // So on every SIMD one wave feeds the matrix cores while the other runs
  // the softmax.  The MFMA phase of tile j reads K(j) and V(j - 1) in slots
  // 2j (A) and 2j + 1 (B); group B copies K(j + 1) and V(j) into the other
  // buffers in slot 2j (at its start in the instances with the vote, at the
  // end of its softmax phase in the dense one), and every wave waits for
  // them at the end of slot 2j + 1.  The dense instance moves the V(j) copy
  // into group A's QK^T steps of slot 2j, so it overlaps MFMA work instead
  // of stretching group B's softmax phase.
  if (tid < kWaves) vote_lds[tid] = -2;
  copy_k(0, lds_k[0], wave);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  const int nslots = 2 * nkt + 2;
  for (int slot = 0; slot < nslots; ++slot) {
    const int my = group_b ? slot - 1 : slot;   // this group's own slot counter
    if constexpr (!kDense) {
      // Group B's copies of K(j + 1) and V(j), at the start of its even slot
      // 2j, before its softmax phase.  Untracked, as in the dense instance:
      // the next slot's MFMA phase reads the other K and V buffers, so it
      // must not wait for these copies (the compiler, seeing an LDS write,
      // would make every operand read wait for them); their one wait is the
      // vmcnt(0) at the end of the odd slot.
      if (group_b && (slot & 1) == 0) {
        const int j = slot >> 1;
        if (j + 1 < nkt) {
          if constexpr (kFp8) {
#pragma unroll
            for (int cj = 0; cj < 4; ++cj)
              copy_one_untracked8(j + 1, lds_k_off + (uint32_t)(((j + 1) & 1) * kTile8Bytes),
                                  2 * (wave - 4) + cj / 2, cj % 2);
          } else {
#pragma unroll
            for (int cj = 0; cj < 2 * kCopyPerWave; ++cj)
              copy_one_untracked(false, j + 1, lds_k_off + (uint32_t)(((j + 1) & 1) * kTileBytes),
                                 2 * (wave - 4) + cj / kCopyPerWave, cj % kCopyPerWave);
          }
        }
        if (j < nkt) {
#pragma unroll
          for (int cj = 0; cj < 2 * kCopyPerWave; ++cj)
            copy_one_untracked(true, j, lds_v_off + (uint32_t)((j & 1) * kTileBytes),
                               2 * (wave - 4) + cj / kCopyPerWave, cj % kCopyPerWave);
        }
      }
    }
    if (my >= 0) {
      const int kt = my >> 1;
      if ((my & 1) == 0) {
        if (kt < nkt) {
          if constexpr (kFp8) {
            if (p_ready)
              mfma_phase8(std::true_type{}, std::true_type{}, kt);
            else
              mfma_phase8(std::false_type{}, std::true_type{}, kt);
          } else if constexpr (kDense) {
            if (p_ready) {
              if (group_b) mfma_phase(std::true_type{}, std::true_type{}, std::false_type{}, kt);
              else mfma_phase(std::true_type{}, std::true_type{}, std::true_type{}, kt);
            } else {
              if (group_b) mfma_phase(std::false_type{}, std::true_type{}, std::false_type{}, kt);
              else mfma_phase(std::false_type{}, std::true_type{}, std::true_type{}, kt);
            }
          } else {
            if (p_ready)
              mfma_phase(std::true_type{}, std::true_type{}, std::false_type{}, kt);
            else
              mfma_phase(std::false_type{}, std::true_type{}, std::false_type{}, kt);
          }
        } else if (p_ready) {
          if constexpr (kFp8)
            mfma_phase8(std::true_type{}, std::false_type{}, kt);
          else
            mfma_phase(std::true_type{}, std::false_type{}, std::false_type{}, kt);
        }
        p_ready = false;
      } else if (kt < nkt) {
        softmax_phase(kt);
      }
    }
    if constexpr (kDense) {
      // The dense instance's K(j + 1) copy, after group B's softmax phase of
      // slot 2j (V(j) was issued by group A during its QK^T steps); the
      // instances with the vote issue theirs at the start of the slot.
      if (group_b && (slot & 1) == 0) {
        const int j = slot >> 1;
        if (j + 1 < nkt) {
#pragma unroll
          for (int cj = 0; cj < 2 * kCopyPerWave; ++cj)
            copy_one_untracked(false, j + 1, lds_k_off + (uint32_t)(((j + 1) & 1) * kTileBytes),
                               2 * (wave - 4) + cj / kCopyPerWave, cj % kCopyPerWave);
        }
      }
    }
    // LDS operations (votes, operand reads) complete before the barrier, so
    // the barrier orders them; a memory fence is not used because it would
    // also wait for copies still in flight.  Copies issued in an even slot
    // are waited for at the end of the following odd slot.
    if (kDebug || (slot & 1) != 0)
      __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
    else
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0) only
    __atomic_signal_fence(__ATOMIC_SEQ_CST);   // no compiler motion of memory operations across the barrier
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }

  // Each vote group's timeout flag, for the epilogue's skip count.
  if (tid < kWaves / 2) vote_timeout[tid] = 0;
  __syncthreads();
  if (timed_out && lane == 0) vote_timeout[wave >> 1] = 1;
  __syncthreads();

  // ---- virtual tiles: add each skipped tile's mean key and value ----
  if constexpr (kComp) {
    const long long tbase = ((long long)b * p.H + h) * nkt;   // this head's first tile
    const uint32_t* my_bits = comp_bits + (wave >> 1) * kCompWords;
    for (int r0 = 0; r0 < nkt; r0 += kCompRound) {
      // Stage kCompRound tiles in the free K/V buffers: for chunk c of 32
      // tiles, mean-key hi rows at 64 c + t and lo rows at 64 c + 32 + t of
      // lds_k (both buffers, 64 KB), mean values at row 32 c + t of lds_v[0]
      // (the tile layouts the operand reads expect).  Tiles past the last one
      // are zero.
      __syncthreads();
      constexpr int kKItems = kCompRound * 2 * 16, kItems = kCompRound * 3 * 16;
#pragma unroll
      for (int it = 0; it < kItems / kThreads; ++it) {
        const int i = tid + kThreads * it;
        const bool isk = i < kKItems;
        const int ii = isk ? i : i - kKItems;
        const int tr = isk ? ii >> 5 : ii >> 4;          // tile within the round
        const int sel = isk ? (ii >> 4) & 1 : 0;          // 0: hi, 1: lo
        const int j = ii & 15;                            // 16-byte chunk of the row
        const int t = r0 + tr;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (t < nkt) {
          const uint16_t* src = isk ? p.kbar + ((tbase + t) * 2 + sel) * kD : p.vbar + (tbase + t) * kD;
          val = *reinterpret_cast<const u32x4*>(src + 8 * j);
        }
        const int row = isk ? 64 * (tr >> 5) + 32 * sel + (tr & 31) : tr;
        unsigned char* dst = (isk ? &lds_k[0][0] : lds_v[0]) + row * kRowBytes + 16 * (j ^ swz(row));
        *reinterpret_cast<u32x4*>(dst) = val;
      }
      __syncthreads();
      for (int c = 0; c < kCompRound / 32 && r0 + 32 * c < nkt; ++c) {
        const int ch = (r0 >> 5) + c;                     // 32-tile word of the skip bits
        const uint32_t bits = my_bits[ch];
        if (bits == 0) continue;                          // this vote group skipped none of them
        const unsigned char* kc = &lds_k[0][0] + 64 * c * kRowBytes;
        const unsigned char* vc = lds_v[0] + 32 * c * kRowBytes;
        // Virtual scores S^T = Kbar Q^T of the 32 tiles (hi and lo parts).
        f32x16 shi = f32x16{}, slo = f32x16{};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int off = krow * kRowBytes + 16 * ((2 * s + hf) ^ kswz);
          const bf16x8 ahi = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kc + off));
          const bf16x8 alo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kc + 32 * kRowBytes + off));
          shi = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, qf[s], shi, 0, 0, 0);
          slo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, qf[s], slo, 0, 0, 0);
        }
        // Weights n_t exp(scale s - r) of this group's skipped tiles, in bf16
        // pairs laid out as the P^T operand; register r holds tile
        // 16 (r / 8) + 8 hf + r % 8 of the chunk.
        uint32_t pw[8];
        float ws = 0.f;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float e[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int tl = 16 * ((r + u) >> 3) + 8 * hf + ((r + u) & 7);
            const int t = 32 * ch + tl;
            e[u] = 0.f;
            if (((bits >> tl) & 1u) != 0 && t < nkt) {
              const int n_t = min(kBK, S_b - kBK * t);
              e[u] = __builtin_amdgcn_exp2f(
                  fmaf(shi[r + u] + slo[r + u], p.scale_log2e, __builtin_amdgcn_logf((float)n_t) - mb_ref));
            }
            ws += e[u];
          }
          pw[r >> 1] = pack_bf16(e[0], e[1]);
        }
        l += ws;
        // O^T += Vbar^T P^T over the 32 tiles (two 16-tile steps).
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const u32x4 pb = {pw[4 * t2], pw[4 * t2 + 1], pw[4 * t2 + 2], pw[4 * t2 + 3]};
          const unsigned char* vstep = vc + 16 * t2 * kRowBytes;
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vstep + voff[0][db]));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vstep + voff[1][db]));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            const u32x4 av = {l2[0], l2[1], h2[0], h2[1]};
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                               __builtin_bit_cast(bf16x8, pb), oacc[db], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- epilogue: O / l in bf16, LSE = r + ln l, skipped-tile count ----
  long long T = 0, qb_off = 0, qb_total = 0;
  if (p.cu_seqlens != nullptr) {
    T = p.cu_seqlens[p.nseq];
    varlen_qblocks(p, b, lane, qb_off, qb_total);
  }
  uint16_t* __restrict__ op = p.o + base;
  const long long ts = p.tok_stride;
  const float lt = halves_sum(l);
  const float inv = 1.f / lt;
  const int row = wrow0 + c;
  if (row < S_b) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 w;
        w.x = pack_bf16(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
        w.y = pack_bf16(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(op + (long long)row * ts + 32 * db + 8 * g + 4 * hf) = w;
      }
    if (p.lse != nullptr && hf == 0) {
      const float lse = mb_ref * (1.f / kLog2e) + logf(lt);
      if (p.cu_seqlens != nullptr)
        p.lse[(long long)h * T + tok0 + row] = lse;
      else
        p.lse[((long long)b * p.H + h) * p.S + row] = lse;
    }
    if (p.maxp != nullptr && hf == 0) {
      // exp(m - LSE) = 1 / l with l taken relative to the row maximum m: the
      // largest weight of the row over the kept keys (clamped to 1, which
      // fp32 rounding of m and of the exponentials can overshoot slightly).
      const float mp = fminf(__builtin_amdgcn_exp2f(m_run * kLog2e - mb_ref) * inv, 1.f);
      if (p.cu_seqlens != nullptr)
        p.maxp[(long long)h * T + tok0 + row] = mp;
      else
        p.maxp[((long long)b * p.H + h) * p.S + row] = mp;
    }
  }
  const long long nqb_seq = (S_b + kBQ - 1) / kBQ;
  if (p.counts != nullptr && lane == 0 && (wave & 1) == 0 && qb < nqb_seq) {
    const int cval = vote_timeout[wave >> 1] != 0 ? -1 - nskip : nskip;
    if (p.cu_seqlens != nullptr) {
      p.counts[(long long)h * qb_total + qb_off + qb] = cval;
    } else {
      const long long nqb = (p.S + kBQ - 1) / kBQ;
      p.counts[((long long)b * p.H + h) * nqb + qb] = cval;
    }
  }
}

// Mean key and mean value of every key tile of a fixed-length [B, H, S, D]
// problem, for the virtual tiles: one workgroup of 256 threads per tile.
// Thread t sums channels 8 (t % 16) .. + 7 over the keys t / 16, t / 16 + 16,
// ... of the tile (16-byte loads, 256 contiguous bytes per key row), in fp32;
// the 16 partial sums of each channel are then added in LDS in a fixed
// order.  The mean key is stored as a bf16 pair hi + lo (hi = bf16(mean),
// lo = bf16(mean - hi)), the mean value as bf16.
__global__ __launch_bounds__(256) void tile_means_kernel(const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v,
                                                           uint16_t* __restrict__ kbar,
                                                           uint16_t* __restrict__ vbar, int H, int S) {
  __shared__ float part[2][16][kD];
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nkt = (S + kBK - 1) / kBK;
  const int g = threadIdx.x & 15, r = threadIdx.x >> 4;
  const long long row0 = ((long long)b * H + h) * S + (long long)t * kBK;
  const int n = min(kBK, S - kBK * t);
#pragma unroll
  for (int isv = 0; isv < 2; ++isv) {
    const uint16_t* src = (isv ? v : k) + row0 * kD + 8 * g;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kBK / 16; ++i) {
      const int key = r + 16 * i;
      if (key < n) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(src + (long long)key * kD);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += __uint_as_float(x[e] << 16);
          acc[2 * e + 1] += __uint_as_float(x[e] & 0xffff0000u);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[isv][r][8 * g + e] = acc[e];
  }
  __syncthreads();
  const int c = threadIdx.x & (kD - 1);
  const int isv = threadIdx.x >> 7;
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) sum += part[isv][i][c];
  const float mean = sum / (float)n;
  const long long tile = ((long long)b * H + h) * nkt + t;
  const uint32_t hi = pack_bf16(mean, 0.f) & 0xffffu;
  if (isv) {
    vbar[tile * kD + c] = (uint16_t)hi;
  } else {
    const float lo = mean - __uint_as_float(hi << 16);
    kbar[(tile * 2) * kD + c] = (uint16_t)hi;
    kbar[(tile * 2 + 1) * kD + c] = (uint16_t)(pack_bf16(lo, 0.f) & 0xffffu);
  }
}

// ---- FP8 (OCP E4M3) quantisation of the score operands -----------------------
// Each value is divided by its block's scale (IEEE float32 division), clamped
// to +-448 and rounded to the nearest E4M3 code (ties to even) by
// v_cvt_pk_fp8_f32.  Scales map the block's largest magnitude to 448:
// scale = amax / 448 (float32 division), or 1 for an all-zero block.
constexpr float kE4m3Max = 448.f;

__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)w, true);
}
__device__ __forceinline__ float clamp448(float x) { return fminf(fmaxf(x, -kE4m3Max), kE4m3Max); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Q: one scale per token.  16 lanes per row, 8 channels per lane.
__global__ __launch_bounds__(256) void quant_q_kernel(const uint16_t* __restrict__ q, uint8_t* __restrict__ q8,
                                                        float* __restrict__ qs, long long rows) {
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int g = threadIdx.x & 15;
  const bool ok = row < rows;
  u32x4 x = {0u, 0u, 0u, 0u};
  if (ok) x = *reinterpret_cast<const u32x4*>(q + row * kD + 8 * g);
  float f[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf16_lo(x[e]);
    f[2 * e + 1] = bf16_hi(x[e]);
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(f[e]));
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));   // within the row's 16 lanes
  const float s = amax > 0.f ? amax / kE4m3Max : 1.f;
  uint2 w;
  w.x = e4m3x4(clamp448(f[0] / s), clamp448(f[1] / s), clamp448(f[2] / s), clamp448(f[3] / s));
  w.y = e4m3x4(clamp448(f[4] / s), clamp448(f[5] / s), clamp448(f[6] / s), clamp448(f[7] / s));
  if (ok) {
    *reinterpret_cast<uint2*>(q8 + row * kD + 8 * g) = w;
    if (g == 0) qs[row] = s;
  }
}

// K: one scale per tile of 128 keys.  One workgroup per tile; lane group
// g = t % 16 holds channels 8 g .. 8 g + 7 of the keys t / 16 + 16 i.
__global__ __launch_bounds__(256) void quant_k_kernel(const uint16_t* __restrict__ k, uint8_t* __restrict__ k8,
                                                        float* __restrict__ ks, int H, int S) {
  __shared__ float red[4];
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nkt = (S + kBK - 1) / kBK;
  const int g = threadIdx.x & 15, r = threadIdx.x >> 4;
  const long long row0 = ((long long)b * H + h) * S + (long long)t * kBK;
  const int n = min(kBK, S - kBK * t);
  u32x4 x[kBK / 16];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kBK / 16; ++i) {
    const int key = r + 16 * i;
    x[i] = u32x4{0u, 0u, 0u, 0u};
    if (key < n) x[i] = *reinterpret_cast<const u32x4*>(k + (row0 + key) * kD + 8 * g);
#pragma unroll
    for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(x[i][e])), fabsf(bf16_hi(x[i][e]))));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax > 0.f ? amax / kE4m3Max : 1.f;
#pragma unroll
  for (int i = 0; i < kBK / 16; ++i) {
    const int key = r + 16 * i;
    uint2 w;
    w.x = e4m3x4(clamp448(bf16_lo(x[i][0]) / s), clamp448(bf16_hi(x[i][0]) / s), clamp448(bf16_lo(x[i][1]) / s),
                 clamp448(bf16_hi(x[i][1]) / s));
    w.y = e4m3x4(clamp448(bf16_lo(x[i][2]) / s), clamp448(bf16_hi(x[i][2]) / s), clamp448(bf16_lo(x[i][3]) / s),
                 clamp448(bf16_hi(x[i][3]) / s));
    if (key < n) *reinterpret_cast<uint2*>(k8 + (row0 + key) * kD + 8 * g) = w;
  }
  if (threadIdx.x == 0) ks[((long long)b * H + h) * nkt + t] = s;
}

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------
thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];   // 0 unknown, 1 gfx950, -1 other
std::atomic<int> g_spin_limit{kSpinLimit};   // polls of the vote exchange (a test hook sets it)
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];                 // device address of `scratch` on each device, once looked up

// The device address of the static workspace on the current device, looked
// up once per device (with that device current) and kept.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(SSA_ERR_DEVICE, "no HIP device is available");
  }
  if (dev >= kMaxDevices) return fail(SSA_ERR_UNSUPPORTED, "device %d beyond the %d this library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return fail(SSA_ERR_LAUNCH, "hipGetSymbolAddress of the static workspace failed on device %d: %s", dev,
                  hipGetErrorString(e));
    }
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return SSA_OK;
}

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(SSA_ERR_DEVICE, "no HIP device is available");
  }
  if (dev < kMaxDevices) {
    const int known = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (known == 1) return SSA_OK;
    if (known == -1) return fail(SSA_ERR_DEVICE, "device %d is not gfx950", dev);
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(SSA_ERR_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
  if (!ok) return fail(SSA_ERR_DEVICE, "device %d is %s, this library runs on gfx950 only", dev, prop.gcnArchName);
  return SSA_OK;
}

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

// Bytes of the virtual-tile workspace: mean keys [B, H, nKT, 2, D] and mean
// values [B, H, nKT, D], bf16.
size_t comp_workspace_bytes(int B, int H, int S) {
  if (B <= 0 || H <= 0 || S <= 0) return 0;
  const size_t nkt = (size_t)((S + kBK - 1) / kBK);
  return (size_t)B * H * nkt * 3 * kD * sizeof(uint16_t);
}

int check_tensors(const void* q, const void* k, const void* v, const void* o, const float* lse, int H, int D, float scale) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr)
    return fail(SSA_ERR_INVALID_ARG, "q, k, v and o must not be NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(SSA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (lse != nullptr && !aligned(lse, 4)) return fail(SSA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (D != kD) return fail(SSA_ERR_UNSUPPORTED, "head dimension %d is not supported (only 128)", D);
  if (H < 0) return fail(SSA_ERR_INVALID_ARG, "negative head count");
  if (H > 65535) return fail(SSA_ERR_UNSUPPORTED, "more than 65535 heads");
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(SSA_ERR_INVALID_ARG, "scale must be finite and positive");
  return SSA_OK;
}

// ln(lambda) for one sequence; lambda computed in double, its log rounded to float.
int resolve(int mode, double p0, double p1, double p2, int seqlen, float* ln_lambda, int* vote) {
  double lam = 0.0;
  switch (mode) {
    case SSA_MODE_FACTOR:
      if (!std::isfinite(p0) || p0 < 0.0) return fail(SSA_ERR_BAD_THRESHOLD, "factor must be finite and >= 0");
      if (seqlen <= 0) return fail(SSA_ERR_BAD_THRESHOLD, "seqlen must be > 0");
      lam = p0 / (double)seqlen;
      break;
    case SSA_MODE_THRESHOLD:
      if (!std::isfinite(p0) || p0 < 0.0) return fail(SSA_ERR_BAD_THRESHOLD, "threshold must be finite and >= 0");
      lam = p0;
      break;
    case SSA_MODE_CALIBRATED: {
      if (!std::isfinite(p0) || !std::isfinite(p1) || !(p0 > 0.0))
        return fail(SSA_ERR_NO_CALIBRATION,
                    "calibrated threshold needs finite coefficients with a > 0; "
                    "without a calibration use the threshold entry (ssa_fwd_threshold)");
      if (!std::isfinite(p2)) return fail(SSA_ERR_BAD_THRESHOLD, "target_sparsity must be finite");
      if (seqlen <= 0) return fail(SSA_ERR_BAD_THRESHOLD, "seqlen must be > 0");
      lam = p0 * std::exp(p1 * p2) / (double)seqlen;
      break;
    }
    default:
      return fail(SSA_ERR_INVALID_ARG, "unknown threshold mode %d", mode);
  }
  if (!std::isfinite(lam) || lam < 0.0) return fail(SSA_ERR_BAD_THRESHOLD, "lambda is not finite");
  *vote = lam > 0.0 ? 1 : 0;
  *ln_lambda = lam > 0.0 ? (float)std::log(lam) : 0.f;
  return SSA_OK;
}

template <bool kDebug, bool kComp = false, bool kFp8 = false>
int launch(const Params& p, dim3 grid, hipStream_t stream) {
  if (!kDebug && !kComp && !kFp8 && p.vote == 0)
    hipLaunchKernelGGL((ssa_fwd_kernel<false, false, false, true>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((ssa_fwd_kernel<kDebug, kComp, kFp8, false>), grid, dim3(kThreads), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SSA_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return SSA_OK;
}

int fwd_fixed(const void* q, const void* k, const void* v, void* o, float* lse, float* maxp, int B, int H, int S,
              int D,
              float scale, int mode, double p0, double p1, double p2, int seqlen, int32_t* counts, uint8_t* mask,
              float* margin, void* stream, bool debug, void* comp_ws = nullptr, size_t comp_ws_bytes = 0,
              bool static_ws = false) {
  int st = check_tensors(q, k, v, o, lse, H, D, scale);
  if (st != SSA_OK) return st;
  if (B < 0 || S < 0) return fail(SSA_ERR_INVALID_ARG, "negative batch or sequence length");
  if (B > 65535) return fail(SSA_ERR_UNSUPPORTED, "batch above 65535");
  // Per-(batch, head) byte offsets, padded to whole tiles, must fit 32 bits.
  if (((long long)S + kBK) * kRowBytes + kRowBytes >= (1LL << 32))
    return fail(SSA_ERR_UNSUPPORTED, "sequence length %d too large", S);
  if (counts != nullptr && !aligned(counts, 4)) return fail(SSA_ERR_INVALID_ARG, "skip_counts must be 4-byte aligned");
  if (margin != nullptr && !aligned(margin, 4)) return fail(SSA_ERR_INVALID_ARG, "tile_margin must be 4-byte aligned");
  if (maxp != nullptr && !aligned(maxp, 4)) return fail(SSA_ERR_INVALID_ARG, "max_prob must be 4-byte aligned");
  if (debug && mask == nullptr) return fail(SSA_ERR_INVALID_ARG, "tile_mask must not be NULL");
  const bool comp = comp_ws != nullptr || static_ws;
  if (comp) {
    if (static_ws) {
      if (comp_workspace_bytes(B, H, S) > kScratchBytes)
        return fail(SSA_ERR_UNSUPPORTED,
                    "the tile means of this call need %zu bytes, above the %zu-byte static workspace "
                    "(B x H x ceil(S / 128) <= %zu); use ssa_fwd_virtual with a workspace",
                    comp_workspace_bytes(B, H, S), kScratchBytes, kScratchBytes / (3 * kD * sizeof(uint16_t)));
    } else {
      if (!aligned(comp_ws, 16)) return fail(SSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
      if (comp_ws_bytes < comp_workspace_bytes(B, H, S))
        return fail(SSA_ERR_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu needed", comp_ws_bytes,
                    comp_workspace_bytes(B, H, S));
    }
    if ((S + kBK - 1) / kBK > 32 * kCompWords)
      return fail(SSA_ERR_UNSUPPORTED, "virtual tiles support at most %d key tiles (S <= %d)", 32 * kCompWords,
                  32 * kCompWords * kBK);
  }
  Params p{};
  st = resolve(mode, p0, p1, p2, seqlen, &p.ln_lambda, &p.vote);
  if (st != SSA_OK) return st;
  if (B == 0 || H == 0 || S == 0) return SSA_OK;
  st = check_device();
  if (st != SSA_OK) return st;
  if (static_ws) {
    st = scratch_address(&comp_ws);
    if (st != SSA_OK) return st;
  }
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.maxp = maxp;
  p.counts = counts;
  p.mask = mask;
  p.margin = margin;
  p.cu_seqlens = nullptr;
  p.nseq = B;
  p.H = H;
  p.S = S;
  p.qgroups = (S + kRowsPerWG - 1) / kRowsPerWG;
  if ((long long)p.qgroups * H * B >= (1LL << 31))
    return fail(SSA_ERR_UNSUPPORTED, "more than 2^31 workgroups (B x H x ceil(S / %d))", kRowsPerWG);
  p.tok_stride = kD;
  p.head_stride = (long long)S * kD;
  p.seq_stride = (long long)H * S * kD;
  p.scale = scale;
  p.scale_log2e = (float)((double)scale * 1.4426950408889634);
  p.lambda_per_seq = 0;
  p.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  const dim3 grid(p.qgroups, H, B);
  if (comp) {
    const int nkt = (S + kBK - 1) / kBK;
    uint16_t* kbar = static_cast<uint16_t*>(comp_ws);
    uint16_t* vbar = kbar + (size_t)B * H * nkt * 2 * kD;
    hipLaunchKernelGGL(tile_means_kernel, dim3(nkt, H, B), dim3(256), 0, static_cast<hipStream_t>(stream),
                       p.k, p.v, kbar, vbar, H, S);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SSA_ERR_LAUNCH, "tile-mean launch failed: %s", hipGetErrorString(e));
    p.kbar = kbar;
    p.vbar = vbar;
    return launch<false, true>(p, grid, static_cast<hipStream_t>(stream));
  }
  return debug ? launch<true>(p, grid, static_cast<hipStream_t>(stream))
               : launch<false>(p, grid, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

int ssa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int S, int D,
            float scale, float factor, int seqlen, int32_t* skip_counts, void* stream) {
  return fwd_fixed(q, k, v, o, lse, nullptr, B, H, S, D, scale, SSA_MODE_FACTOR, factor, 0.0, 0.0, seqlen, skip_counts,
                   nullptr, nullptr, stream, false);
}

int ssa_fwd_threshold(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int S, int D,
                      float scale, float threshold, int32_t* skip_counts, void* stream) {
  return fwd_fixed(q, k, v, o, lse, nullptr, B, H, S, D, scale, SSA_MODE_THRESHOLD, threshold, 0.0, 0.0, S, skip_counts,
                   nullptr, nullptr, stream, false);
}

int ssa_fwd_calibrated(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int S,
                       int D, float scale, float a, float b, float target_sparsity, int seqlen, int32_t* skip_counts,
                       void* stream) {
  return fwd_fixed(q, k, v, o, lse, nullptr, B, H, S, D, scale, SSA_MODE_CALIBRATED, a, b, target_sparsity, seqlen,
                   skip_counts, nullptr, nullptr, stream, false);
}

int ssa_fwd_debug(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int S, int D,
                  float scale, int mode, double p0, double p1, double p2, int seqlen, int32_t* skip_counts,
                  uint8_t* tile_mask, float* tile_margin, void* stream) {
  return fwd_fixed(q, k, v, o, lse, nullptr, B, H, S, D, scale, mode, p0, p1, p2, seqlen, skip_counts, tile_mask,
                   tile_margin, stream, true);
}

int ssa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int S, int D,
               float scale, int mode, double p0, double p1, double p2, int seqlen, int32_t* skip_counts,
               float* max_prob, void* stream) {
  return fwd_fixed(q, k, v, o, lse, max_prob, B, H, S, D, scale, mode, p0, p1, p2, seqlen, skip_counts, nullptr,
                   nullptr, stream, false);
}

size_t ssa_fwd_virtual_workspace_bytes(int B, int H, int S) { return comp_workspace_bytes(B, H, S); }

int ssa_fwd_virtual(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int S, int D,
                    float scale, int mode, double p0, double p1, double p2, int seqlen, int32_t* skip_counts,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace == nullptr) return fail(SSA_ERR_INVALID_ARG, "workspace must not be NULL");
  return fwd_fixed(q, k, v, o, lse, nullptr, B, H, S, D, scale, mode, p0, p1, p2, seqlen, skip_counts, nullptr,
                   nullptr, stream, false, workspace, workspace_bytes);
}

int ssa_fwd_virtual_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int S,
                            int D, float scale, int mode, double p0, double p1, double p2, int seqlen,
                            int32_t* skip_counts, void* stream) {
  return fwd_fixed(q, k, v, o, lse, nullptr, B, H, S, D, scale, mode, p0, p1, p2, seqlen, skip_counts, nullptr,
                   nullptr, stream, false, nullptr, 0, true);
}

int ssa_quantize_qk_fp8(const void* q, const void* k, uint8_t* q8, uint8_t* k8, float* q_scale, float* k_scale,
                        int B, int H, int S, int D, void* stream) {
  if (q == nullptr || k == nullptr || q8 == nullptr || k8 == nullptr || q_scale == nullptr || k_scale == nullptr)
    return fail(SSA_ERR_INVALID_ARG, "q, k, q8, k8, q_scale and k_scale must not be NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(q8, 8) || !aligned(k8, 8) || !aligned(q_scale, 4) ||
      !aligned(k_scale, 4))
    return fail(SSA_ERR_INVALID_ARG, "q, k must be 16-byte, q8, k8 8-byte and the scales 4-byte aligned");
  if (D != kD) return fail(SSA_ERR_UNSUPPORTED, "head dimension %d is not supported (only 128)", D);
  if (B < 0 || H < 0 || S < 0) return fail(SSA_ERR_INVALID_ARG, "negative batch, head count or length");
  if (B > 65535 || H > 65535) return fail(SSA_ERR_UNSUPPORTED, "batch or head count above 65535");
  if (B == 0 || H == 0 || S == 0) return SSA_OK;
  const int st = check_device();
  if (st != SSA_OK) return st;
  const long long rows = (long long)B * H * S;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(quant_q_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(q), q8, q_scale, rows);
  hipLaunchKernelGGL(quant_k_kernel, dim3((S + kBK - 1) / kBK, H, B), dim3(256), 0, s,
                     static_cast<const uint16_t*>(k), k8, k_scale, H, S);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SSA_ERR_LAUNCH, "quantisation launch failed: %s", hipGetErrorString(e));
  return SSA_OK;
}

int ssa_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const float* q_scale, const float* k_scale, const void* v,
                void* o, float* lse, int B, int H, int S, int D, float scale, int mode, double p0, double p1,
                double p2, int seqlen, int32_t* skip_counts, uint8_t* tile_mask, float* tile_margin, void* stream) {
  if (q8 == nullptr || k8 == nullptr || q_scale == nullptr || k_scale == nullptr)
    return fail(SSA_ERR_INVALID_ARG, "q8, k8, q_scale and k_scale must not be NULL");
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(q_scale, 4) || !aligned(k_scale, 4))
    return fail(SSA_ERR_INVALID_ARG, "q8, k8 must be 16-byte and the scales 4-byte aligned");
  int st = check_tensors(v, v, v, o, lse, H, D, scale);
  if (st != SSA_OK) return st;
  if (B < 0 || S < 0) return fail(SSA_ERR_INVALID_ARG, "negative batch or sequence length");
  if (B > 65535) return fail(SSA_ERR_UNSUPPORTED, "batch above 65535");
  if (((long long)S + kBK) * kRowBytes + kRowBytes >= (1LL << 32))
    return fail(SSA_ERR_UNSUPPORTED, "sequence length %d too large", S);
  if ((S + kBK - 1) / kBK > kMaxTilesFp8)
    return fail(SSA_ERR_UNSUPPORTED, "FP8 scores support at most %d key tiles (S <= %d)", kMaxTilesFp8,
                kMaxTilesFp8 * kBK);
  if (skip_counts != nullptr && !aligned(skip_counts, 4)) return fail(SSA_ERR_INVALID_ARG, "skip_counts must be 4-byte aligned");
  if (tile_margin != nullptr && !aligned(tile_margin, 4)) return fail(SSA_ERR_INVALID_ARG, "tile_margin must be 4-byte aligned");
  if (tile_margin != nullptr && tile_mask == nullptr) return fail(SSA_ERR_INVALID_ARG, "tile_margin needs tile_mask");
  Params p{};
  st = resolve(mode, p0, p1, p2, seqlen, &p.ln_lambda, &p.vote);
  if (st != SSA_OK) return st;
  if (B == 0 || H == 0 || S == 0) return SSA_OK;
  st = check_device();
  if (st != SSA_OK) return st;
  p.q = static_cast<const uint16_t*>(v);   // bf16 Q and K are not read on this path
  p.k = static_cast<const uint16_t*>(v);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.q8 = q8;
  p.k8 = k8;
  p.q_scale = q_scale;
  p.k_scale = k_scale;
  p.lse = lse;
  p.counts = skip_counts;
  p.mask = tile_mask;
  p.margin = tile_margin;
  p.nseq = B;
  p.H = H;
  p.S = S;
  p.qgroups = (S + kRowsPerWG - 1) / kRowsPerWG;
  if ((long long)p.qgroups * H * B >= (1LL << 31))
    return fail(SSA_ERR_UNSUPPORTED, "more than 2^31 workgroups (B x H x ceil(S / %d))", kRowsPerWG);
  p.tok_stride = kD;
  p.head_stride = (long long)S * kD;
  p.seq_stride = (long long)H * S * kD;
  p.scale = scale;
  p.scale_log2e = (float)((double)scale * 1.4426950408889634);
  p.lambda_per_seq = 0;
  p.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  const dim3 grid(p.qgroups, H, B);
  return tile_mask != nullptr ? launch<true, false, true>(p, grid, static_cast<hipStream_t>(stream))
                              : launch<false, false, true>(p, grid, static_cast<hipStream_t>(stream));
}

int ssa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens,
                   int nseq, int max_seqlen, int H, int D, float scale, int mode, double p0, double p1, double p2,
                   int32_t* skip_counts, void* stream) {
  int st = check_tensors(q, k, v, o, lse, H, D, scale);
  if (st != SSA_OK) return st;
  if (cu_seqlens == nullptr || !aligned(cu_seqlens, 4)) return fail(SSA_ERR_INVALID_ARG, "cu_seqlens must be a 4-byte aligned device pointer");
  if (nseq < 0 || max_seqlen < 0) return fail(SSA_ERR_INVALID_ARG, "negative nseq or max_seqlen");
  if (nseq > 65535) return fail(SSA_ERR_UNSUPPORTED, "more than 65535 sequences");
  if (((long long)max_seqlen + kBK) * H * kRowBytes + kRowBytes >= (1LL << 32))
    return fail(SSA_ERR_UNSUPPORTED, "max_seqlen x heads too large for 32-bit offsets");
  if (skip_counts != nullptr && !aligned(skip_counts, 4)) return fail(SSA_ERR_INVALID_ARG, "skip_counts must be 4-byte aligned");
  Params p{};
  // Validate the control once with a representative length; the kernel
  // recomputes ln(lambda_b) for each sequence's own length.
  st = resolve(mode, p0, p1, p2, max_seqlen > 0 ? max_seqlen : 1, &p.ln_lambda, &p.vote);
  if (st != SSA_OK) return st;
  if (nseq == 0 || H == 0 || max_seqlen == 0) return SSA_OK;
  st = check_device();
  if (st != SSA_OK) return st;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.counts = skip_counts;
  p.cu_seqlens = cu_seqlens;
  p.nseq = nseq;
  p.H = H;
  p.S = max_seqlen;
  p.qgroups = (max_seqlen + kRowsPerWG - 1) / kRowsPerWG;
  if ((long long)p.qgroups * H * nseq >= (1LL << 31))
    return fail(SSA_ERR_UNSUPPORTED, "more than 2^31 workgroups (nseq x H x ceil(max_seqlen / %d))", kRowsPerWG);
  p.tok_stride = (long long)H * kD;
  p.head_stride = kD;
  p.seq_stride = 0;
  p.scale = scale;
  p.scale_log2e = (float)((double)scale * 1.4426950408889634);
  p.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  if (mode == SSA_MODE_THRESHOLD) {
    p.lambda_per_seq = 0;
  } else {
    p.lambda_per_seq = 1;
    p.factor = mode == SSA_MODE_FACTOR ? p0 : p0 * std::exp(p1 * p2);
  }
  // 8 XCD lists, each long enough for an eighth (rounded up) of every
  // sequence's H * qgroups items.
  const long long per_xcd = (long long)nseq * (((long long)H * p.qgroups + kXcds - 1) / kXcds);
  if (per_xcd * kXcds >= (1LL << 31))
    return fail(SSA_ERR_UNSUPPORTED, "more than 2^31 workgroups (nseq x H x ceil(max_seqlen / %d))", kRowsPerWG);
  const dim3 grid((unsigned)(per_xcd * kXcds));
  return launch<false>(p, grid, static_cast<hipStream_t>(stream));
}

int ssa_resolve_threshold(int mode, double p0, double p1, double p2, int seqlen, float* ln_lambda,
                          int* vote_enabled) {
  if (ln_lambda == nullptr || vote_enabled == nullptr) return fail(SSA_ERR_INVALID_ARG, "NULL output pointer");
  return resolve(mode, p0, p1, p2, seqlen, ln_lambda, vote_enabled);
}

int ssa_device_check(void) { return check_device(); }

int ssa_set_vote_poll_limit(int polls) {
  if (polls < 0 || polls > kMaxSpinLimit)
    return fail(SSA_ERR_INVALID_ARG, "vote poll limit %d outside [0, %d]", polls, kMaxSpinLimit);
  g_spin_limit.store(polls, std::memory_order_relaxed);
  return SSA_OK;
}

int ssa_vote_poll_limit(void) { return g_spin_limit.load(std::memory_order_relaxed); }

const char* ssa_strerror(int status) {
  switch (status) {
    case SSA_OK: return "SSA_OK";
    case SSA_ERR_INVALID_ARG: return "SSA_ERR_INVALID_ARG: invalid argument";
    case SSA_ERR_UNSUPPORTED: return "SSA_ERR_UNSUPPORTED: unsupported shape";
    case SSA_ERR_BAD_THRESHOLD: return "SSA_ERR_BAD_THRESHOLD: threshold, factor or seqlen out of range";
    case SSA_ERR_NO_CALIBRATION: return "SSA_ERR_NO_CALIBRATION: missing calibration, use the threshold entry";
    case SSA_ERR_DEVICE: return "SSA_ERR_DEVICE: no gfx950 device";
    case SSA_ERR_LAUNCH: return "SSA_ERR_LAUNCH: kernel launch failed";
    case SSA_ERR_BAD_CONFIG: return "SSA_ERR_BAD_CONFIG: unsupported calibration formula";
    default: return "unknown ssa_status";
  }
}

const char* ssa_last_error(void) { return g_last_error; }

int ssa_version(void) { return 1; }

}  // extern "C"
