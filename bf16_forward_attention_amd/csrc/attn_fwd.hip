// attn_fwd.hip -- fused non-causal bf16 forward attention for MI355X (gfx950).
//
// O = softmax(Q K^T / sqrt(128)) V per (batch, head, query row), the
// operation the snilld.dk page "Open source attention kernel in HIP beats
// AITER v3 on MI300X" describes (section "Hvordan kernen arbejder" / How the
// kernel works), streamed over key tiles with a running maximum and sum so
// the score matrix never leaves registers (the FlashAttention family the same
// page places the design in, section "Memory-placement og mikroarkitektur").
//
// Work decomposition.  One workgroup of 8 wave64s (two per SIMD) owns
// BM = 256 query rows of one (batch, head); each wave owns 32 of them.  Keys
// stream in tiles of BN = 64, shared through LDS by all eight waves.  Both products run on v_mfma_f32_32x32x16_bf16 in the transposed
// orientation
//     S^T (keys x queries)  = K   . Q^T      A = K tile (LDS), B = Q (VGPRs)
//     O^T (dims x queries) += V^T . P^T      A = V tile read transposed (LDS), B = P (VGPRs)
// so that every lane owns exactly one query row: the softmax row statistics
// are per-lane scalars plus one exchange between the two 32-lane halves, and
// the rescale of the output accumulator is a per-lane multiply.
//
// MFMA 32x32x16 operand layout (lane l, g = l / 32):
//     A[i][k]: lane supplies row i = l % 32, k = 8g .. 8g+7
//     B[k][j]: lane supplies column j = l % 32, k = 8g .. 8g+7
//     C[i][j]: lane holds column j = l % 32, rows 8r + 4g + t in element 4r + t
//
// Data movement.  K and V tiles go from HBM straight into LDS with
// buffer_load_dwordx4 ... lds (lane l of a load lands at 16*l past the
// wave's LDS base), four stages deep with loads issued three tiles ahead
// (one tile of lead leaves the matrix cores waiting on load latency), one
// workgroup barrier per tile.  The
// buffer descriptor of each tile ends at the last valid key, so keys past Sk
// read as zeros without any per-lane test.  LDS rows are 256 bytes, with the
// 16-byte chunks XOR-swizzled by row so the MFMA operand reads are free of
// bank conflicts on gfx950's 64-bank LDS (16 lanes per cycle for 16-byte
// reads, 32 lanes per cycle for 8-byte reads): K chunk c of row r sits at
// c ^ (r % 16), V chunk c of row r at c ^ 4(r % 4).
//
// Key order inside a 32-key block.  LDS K row i holds key
// pi(i) = 16*(i/4 % 2) + 4*(i/8) + i%4, so that after the first product lane
// group g holds the 16 consecutive keys 16g .. 16g+15 of the block in
// elements 0..15.  Eight of those are exactly a B operand of the second
// product; the matching A operand (8 consecutive keys of one V column) comes
// from two ds_read_b64_tr_b16 reads of the row-major V tile.  Within each
// 16-lane group that instruction hands lane i element i%4 of the 8-byte
// chunks addressed by lanes 4s + i/4 (s = 0..3); pointing lane 4s + u at keys
// key0 + s, dims dim0 + 4u .. 4u+3 gives lane i the four keys key0 .. key0+3
// at dim dim0 + i.
//
// Numerics.  Logits accumulate in fp32 on the matrix cores.  The softmax runs
// in the base-2 domain: t = s * log2(e)/sqrt(128) (one fp32 constant), the
// running maximum m starts at -FLT_MAX (finite, so an all -Inf prefix never
// forms -Inf - -Inf) and is kept rounded up so the maximal key's weight is
// never above 1, p = exp2(t - m) on the hardware exp, the row sum l in fp32
// from the unrounded p.  The maximum (and with it the accumulator) is only
// moved when some row's maximum grew by more than 2^8: between moves the
// weights stay below 256, which fp32 and bf16 carry without loss of relative
// precision.  P is rounded to bf16 (nearest-even) for the second product.
// The epilogue multiplies by 1/l and rounds once to bf16 in the requested
// mode.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "attn_fwd.h"

namespace {

constexpr int D = 128;
constexpr int BM = 256;                // query rows per workgroup
constexpr int BN = 64;                 // keys per tile
constexpr int NWAVES = BM / 32;        // 32 query rows per wave: 8 waves, two per SIMD
constexpr int NTHREADS = NWAVES * 64;
constexpr int TILE_BYTES = BN * D * 2; // one K or V tile in LDS (16 KiB)
constexpr int NSTAGE = 4;              // LDS stages: tiles are loaded three ahead
constexpr float kRescaleLog2 = 8.0f;   // move the running maximum only past 2^8

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;
// log2(e) / sqrt(128), rounded to fp32
constexpr float kScaleLog2 = 0.12751743082459868f;
// gfx9 buffer descriptor word 3: 32-bit data format, no swizzle, raw addressing
constexpr int kBufferWord3 = 0x00020000;

struct Geometry {
  int64_t q_row;   // element stride between consecutive query rows
  int64_t k_row;   // element stride between consecutive key rows
  int64_t q_head;  // element offset of head h within batch b: q_head * h
  int64_t k_head;
  int64_t q_batch; // element offset of batch b
  int64_t k_batch;
};

// Combine a per-lane value with the one held 32 lanes away (the other half of
// the wave).  This goes through ds_bpermute: AMD clang 22 folds
// fmaxf(r[0], r[1]) of __builtin_amdgcn_permlane32_swap(x, x) into r[0], as
// if the swap of a register with itself were the identity, which leaves the
// two halves with different values.
__device__ __forceinline__ float wave_half_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
// fp32 addition is commutative, so both halves get identical bits
__device__ __forceinline__ float wave_half_sum(float x) { return x + __shfl_xor(x, 32); }

template <int MODE>
__device__ __forceinline__ uint16_t round_to_bf16(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if (MODE == ATTN_ROUND_RTNE) {
    __bf16 b = (__bf16)x;  // v_cvt_pk_bf16_f32: nearest-even, NaN stays NaN
    return __builtin_bit_cast(uint16_t, b);
  }
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;  // NaN: canonical quiet NaN
  if (MODE == ATTN_ROUND_RTNA) return (uint16_t)((u + 0x8000u) >> 16);
  return (uint16_t)(u >> 16);  // RTZ
}

// pi within a 32-key block: LDS row -> key
__device__ __forceinline__ int key_of_k_row(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: 48-bit base, stride 0, num_records bytes, word 3.
// All four words are wave-uniform (scalar registers).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t num_records) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(a >> 32) & 0xFFFF);
  r[2] = __builtin_amdgcn_readfirstlane((int32_t)num_records);
  r[3] = kBufferWord3;
  return r;
}

// One direct-to-LDS load: 16 bytes per lane from rsrc + voffset land at
// lds_base + 16 * lane.  Written as a single-instruction asm wrapper (plus
// the M0 set-up and the one-cycle M0 hazard wait) so the compiler does not
// track it as an LDS write: it would otherwise wait for every such load in
// flight before each later LDS read, since it cannot tell which stage a load
// fills.  The kernel orders these loads itself with s_waitcnt vmcnt and the
// workgroup barrier (loads complete in order).  M0 is a reserved register
// that the compiler itself sets right before each of its own uses.
__device__ __forceinline__ void lds_dma_b128(i32x4 rsrc, uint32_t lds_base, uint32_t voffset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voffset), "s"(rsrc)
               : "memory");
}

// LDS address (offset within the workgroup's LDS) of a __shared__ pointer
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

template <int MODE>
__global__ __launch_bounds__(NTHREADS, 1) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, int H, int Sq, int Sk, int n_qtiles, Geometry g) {
  // one array per stage, so the compiler can tell the stages apart when it
  // places waits for the direct-to-LDS loads
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds2[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds3[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds2[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds3[TILE_BYTES];
  uint8_t* const k_st[NSTAGE] = {k_lds0, k_lds1, k_lds2, k_lds3};
  uint8_t* const v_st[NSTAGE] = {v_lds0, v_lds1, v_lds2, v_lds3};

  // ---- workgroup -> (b, h, q-tile), keeping a head's q-tiles on one XCD ----
  // Workgroups are dispatched round-robin over the 8 XCDs; renumber so that
  // XCD x receives a contiguous range of logical work items.
  const int nwg = gridDim.x;
  const int id = blockIdx.x;
  const int xcd = id & 7, local = id >> 3;
  const int per = nwg >> 3, rem = nwg & 7;
  const int work = xcd * per + (xcd < rem ? xcd : rem) + local;
  const int qt = work % n_qtiles;
  const int bh = work / n_qtiles;
  const int h = bh % H, b = bh / H;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int grp = lane >> 5;

  const uint16_t* Qh = Q + b * g.q_batch + h * g.q_head;
  const uint16_t* Kh = K + b * g.k_batch + h * g.k_head;
  const uint16_t* Vh = V + b * g.k_batch + h * g.k_head;
  uint16_t* Oh = O + b * g.q_batch + h * g.q_head;
  const uint32_t row_bytes = (uint32_t)(g.k_row * 2);

  // ---- Q fragments: this lane's query row, dims 16ks + 8grp .. +7 ----
  const int qrow = qt * BM + wave * 32 + l32;
  bf16x8 qf[8];
  {
    const bool ok = qrow < Sq;
    const uint16_t* src = Qh + (int64_t)(ok ? qrow : 0) * g.q_row + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 w = ok ? *(const u32x4*)(src + 16 * ks) : u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }
  // Q must be in registers before the tile loop: the compiler cannot see the
  // direct-to-LDS loads and would otherwise re-wait for Q inside the loop,
  // draining the tile loads in flight with it.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // ---- direct-to-LDS load assignment: wave w issues loads j = 2w + u ----
  // Load j fills LDS rows 4j .. 4j+3 (1 KiB); lane l writes row 4j + l/16 at
  // 16-byte position l%16, which holds logical chunk (l%16) ^ swizzle(row).
  uint32_t k_src[2], v_src[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = 4 * (2 * wave + u) + (lane >> 4);
    const int p = lane & 15;
    const int kc = p ^ (r & 15);
    const int key = (r & 32) + key_of_k_row(r & 31);
    k_src[u] = (uint32_t)key * row_bytes + 16u * kc;
    const int vc = p ^ (4 * (r & 3));
    v_src[u] = (uint32_t)r * row_bytes + 16u * vc;
  }

  // ---- MFMA operand read offsets (bytes within a tile) ----
  // K: row l32 (+32 kb), logical chunk 2ks + grp at position chunk ^ (row % 16)
  uint32_t k_rd[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) k_rd[ks] = 256u * l32 + 16u * ((2 * ks + grp) ^ (l32 & 15));
  // V (transposed reads): lane 16G + 4s + u reads keys 16(G/2) + 4half + s
  // (+32kb + 8hh), dims 32db + 16(G%2) + 4u .. +3, logical chunk
  // 4db + 2(G%2) + u/2 at position chunk ^ (4 * (row % 4))
  uint32_t v_rd[4][2];
  {
    const int G = lane >> 4, sidx = (lane >> 2) & 3, u4 = lane & 3;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int row = 16 * (G >> 1) + 4 * half + sidx;
        const int chunk = 4 * db + 2 * (G & 1) + (u4 >> 1);
        v_rd[db][half] = 256u * row + 16u * (chunk ^ (4 * (row & 3))) + 8u * (u4 & 1);
      }
  }

  auto issue_loads = [&](int tile, uint8_t* kdst, uint8_t* vdst) __attribute__((always_inline)) {
    const int base = tile * BN;
    const int valid = Sk - base < BN ? Sk - base : BN;
    const uint32_t nrec = (uint32_t)(valid - 1) * row_bytes + 256u;
    const i32x4 rk = make_rsrc(Kh + (int64_t)base * g.k_row, nrec);
    const i32x4 rv = make_rsrc(Vh + (int64_t)base * g.k_row, nrec);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = 2 * wave + u;
      lds_dma_b128(rk, __builtin_amdgcn_readfirstlane(lds_addr(kdst + 1024 * j)), k_src[u]);
      lds_dma_b128(rv, __builtin_amdgcn_readfirstlane(lds_addr(vdst + 1024 * j)), v_src[u]);
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
  float m_run = -3.402823466e38f;
  float l_run = 0.0f;

  const int n_tiles = (Sk + BN - 1) / BN;

  auto compute_tile = [&](int t, const uint8_t* kt, const uint8_t* vt) __attribute__((always_inline)) {
    const int base = t * BN;
    // ---- S^T = K . Q^T for the two 32-key blocks ----
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        bf16x8 a = *(const bf16x8*)(kt + k_rd[ks] + 8192 * kb);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
      }
    // read K operands four MFMAs ahead of their use (the compiler otherwise
    // issues each read just before its MFMA and the matrix core waits on LDS)
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);

    // keys past Sk (only in the last tile) get a -Inf logit
    if (base + BN > Sk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int n = 0; n < 16; ++n)
          if (base + 32 * kb + 16 * grp + n >= Sk) s[kb][n] = -__builtin_inff();
    }

    // ---- online softmax (base 2) ----
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int n = 0; n < 16; ++n) mx = fmaxf(mx, s[kb][n]);
    mx = wave_half_max(mx);
    // The candidate maximum is the scaled row maximum rounded up by at least
    // half an ulp: then fma(s, c, -m) <= 0 for the maximal logit, its weight
    // is exp2(<= 0) <= 1 and rounds to exactly 1 in bf16, so a row dominated
    // by one key (or with a single key) returns that V row exactly in every
    // mode.  (-Inf / NaN maxima give NaN here, which fmaxf ignores.)
    const float mx_scaled = mx * kScaleLog2;
    const float m_new = fmaxf(m_run, __builtin_fmaf(__builtin_fabsf(mx_scaled), 0x1p-23f, mx_scaled));
    if (__builtin_amdgcn_ballot_w64(m_new > m_run + kRescaleLog2) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] *= alpha;
    }

    float psum = 0.0f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const int n = 8 * hh + 2 * q2;
          f32x2 p;
          p[0] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][n], kScaleLog2, -m_run));
          p[1] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][n + 1], kScaleLog2, -m_run));
          psum += p[0];
          psum += p[1];
          bf16x2 pb = __builtin_convertvector(p, bf16x2);
          pf[kb][hh][2 * q2] = pb[0];
          pf[kb][hh][2 * q2 + 1] = pb[1];
        }
      }
    }
    l_run += psum;

    // ---- O^T += V^T . P^T ----
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const uint8_t* vb = vt + 256 * (32 * kb + 8 * hh);
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vb + v_rd[db][0]));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vb + v_rd[db][1]));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kb][hh], acc[db], 0, 0, 0);
        }
    // V operands (two transposed reads each) four MFMAs ahead of their use
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
  };

  // ---- main loop: four LDS stages, tiles loaded three ahead, one barrier per tile ----
  // Tile t lives in stage t % 4.  Before computing tile t a wave waits until
  // its own loads of tile t have landed (loads complete in order, so the
  // four loads of each later tile in flight may remain outstanding), then
  // the barrier makes every wave's loads visible and guarantees that stage
  // (t+3) % 4, last read for tile t-1, is free for the loads of tile t+3.
  auto step = [&](auto st_c, int t) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value;
    if (t + 2 < n_tiles)
      __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8): tiles t+1 and t+2 may still be in flight
    else if (t + 1 < n_tiles)
      __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (t + 3 < n_tiles) issue_loads(t + 3, k_st[(ST + 3) % NSTAGE], v_st[(ST + 3) % NSTAGE]);
    compute_tile(t, k_st[ST], v_st[ST]);
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  issue_loads(0, k_lds0, v_lds0);
  if (n_tiles > 1) issue_loads(1, k_lds1, v_lds1);
  if (n_tiles > 2) issue_loads(2, k_lds2, v_lds2);
  for (int t = 0; t < n_tiles; t += 4) {
    step(S0{}, t);
    if (t + 1 < n_tiles) step(S1{}, t + 1);
    if (t + 2 < n_tiles) step(S2{}, t + 2);
    if (t + 3 < n_tiles) step(S3{}, t + 3);
  }

  // ---- epilogue: normalise, round, store this lane's query row ----
  const float l_tot = wave_half_sum(l_run);
  const float inv_l = 1.0f / l_tot;
  if (qrow < Sq) {
    uint16_t* dst = Oh + (int64_t)qrow * g.q_row + 4 * grp;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t lo = round_to_bf16<MODE>(acc[db][4 * r + 0] * inv_l) |
                      ((uint32_t)round_to_bf16<MODE>(acc[db][4 * r + 1] * inv_l) << 16);
        uint32_t hi = round_to_bf16<MODE>(acc[db][4 * r + 2] * inv_l) |
                      ((uint32_t)round_to_bf16<MODE>(acc[db][4 * r + 3] * inv_l) << 16);
        *(u32x2*)(dst + 32 * db + 8 * r) = u32x2{lo, hi};
      }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ERR_DEVICE;
  if (dev < kMaxDevices) {
    int st = g_arch_state[dev].load(std::memory_order_acquire);
    if (st == 1) return ATTN_OK;
    if (st == 2) return ATTN_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_state[dev].store(ok ? 1 : 2, std::memory_order_release);
  return ok ? ATTN_OK : ATTN_ERR_DEVICE;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

}  // namespace

extern "C" int attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H,
                             int64_t Sq, int64_t Sk, int layout, int round_mode, void* stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1) return ATTN_ERR_SIZE;
  int64_t bh, nq, nk, bytes_q, bytes_k;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, Sq, &nq) || !mul_ok(nq, 2 * D, &bytes_q) || !mul_ok(bh, Sk, &nk) ||
      !mul_ok(nk, 2 * D, &bytes_k))
    return ATTN_ERR_SIZE;
  const int64_t n_qtiles = (Sq + BM - 1) / BM;
  int64_t n_wg;
  // one 64-key tile of rows must be addressable by 32-bit buffer offsets
  if (!mul_ok(bh, n_qtiles, &n_wg) || n_wg > INT32_MAX || Sq > INT32_MAX || Sk > INT32_MAX || H > (1 << 20))
    return ATTN_ERR_SIZE;
  if (layout != ATTN_LAYOUT_BSHD && layout != ATTN_LAYOUT_BHSD) return ATTN_ERR_LAYOUT;
  if (round_mode != ATTN_ROUND_RTNE && round_mode != ATTN_ROUND_RTNA && round_mode != ATTN_ROUND_RTZ)
    return ATTN_ERR_ROUND;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return ATTN_ERR_ALIGN;
  if (overlaps(o, bytes_q, q, bytes_q) || overlaps(o, bytes_q, k, bytes_k) || overlaps(o, bytes_q, v, bytes_k))
    return ATTN_ERR_ALIAS;
  const int dev_status = check_device();
  if (dev_status != ATTN_OK) return dev_status;

  Geometry g;
  if (layout == ATTN_LAYOUT_BSHD) {
    g.q_row = H * D;
    g.k_row = H * D;
    g.q_head = D;
    g.k_head = D;
    g.q_batch = Sq * H * D;
    g.k_batch = Sk * H * D;
  } else {
    g.q_row = D;
    g.k_row = D;
    g.q_head = Sq * D;
    g.k_head = Sk * D;
    g.q_batch = H * Sq * D;
    g.k_batch = H * Sk * D;
  }
  const dim3 grid((unsigned)n_wg), block(NTHREADS);
  hipStream_t s = (hipStream_t)stream;
  const uint16_t *qq = (const uint16_t*)q, *kk = (const uint16_t*)k, *vv = (const uint16_t*)v;
  uint16_t* oo = (uint16_t*)o;
  switch (round_mode) {
    case ATTN_ROUND_RTNE:
      hipLaunchKernelGGL(attn_fwd_kernel<ATTN_ROUND_RTNE>, grid, block, 0, s, qq, kk, vv, oo, (int)H, (int)Sq,
                         (int)Sk, (int)n_qtiles, g);
      break;
    case ATTN_ROUND_RTNA:
      hipLaunchKernelGGL(attn_fwd_kernel<ATTN_ROUND_RTNA>, grid, block, 0, s, qq, kk, vv, oo, (int)H, (int)Sq,
                         (int)Sk, (int)n_qtiles, g);
      break;
    default:
      hipLaunchKernelGGL(attn_fwd_kernel<ATTN_ROUND_RTZ>, grid, block, 0, s, qq, kk, vv, oo, (int)H, (int)Sq,
                         (int)Sk, (int)n_qtiles, g);
      break;
  }
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" const char* attn_fwd_bf16_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL: return "a tensor pointer is NULL";
    case ATTN_ERR_SIZE: return "B, H, Sq and Sk must be >= 1 and the problem must fit the index types";
    case ATTN_ERR_LAYOUT: return "layout must be ATTN_LAYOUT_BSHD or ATTN_LAYOUT_BHSD";
    case ATTN_ERR_ROUND: return "round_mode must be ATTN_ROUND_RTNE, ATTN_ROUND_RTNA or ATTN_ROUND_RTZ";
    case ATTN_ERR_ALIGN: return "q, k, v and o must be 16-byte aligned";
    case ATTN_ERR_ALIAS: return "o overlaps q, k or v";
    case ATTN_ERR_DEVICE: return "the current HIP device is not gfx950 (MI355X) or cannot be queried";
    case ATTN_ERR_HIP: return "the HIP kernel launch failed";
    default: return "unknown status";
  }
}

extern "C" int attn_fwd_bf16_abi_version(void) { return ATTN_FWD_ABI_VERSION; }
