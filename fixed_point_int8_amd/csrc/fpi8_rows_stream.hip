// fpi8_rows_stream.hip - the standalone matrix row over many rows ("A matrix
// row" of "The inference core" page): y = ((sum_c w_c x_c - 128 sum_c x_c)
// * scale) >> 24 in wrapping 64-bit arithmetic, for a matrix of packed
// operand tiles with enough rows to give every compute unit many tiles.
//
// The arithmetic is that of the other row kernels: three signed base-256
// digits of each input word on the int8 matrix cores, the weight byte's top
// bit flipped to make it the signed weight, exact i32 partial sums
// recombined in i64 (equal to the page's form modulo 2^64).  What differs
// is the schedule, built for a launch that streams far more weight bytes
// than the last-level cache holds:
//
//  * Workgroups are persistent: one (or a few) per compute unit, each
//    walking its share of the row tiles.  A wave's prefetch ring runs
//    straight across tile boundaries, so the weight stream never drains
//    between tiles; the epilogue of a tile overlaps the next tile's loads.
//  * Weight tiles are read with nontemporal loads (each byte is used once).
//  * k_rows_stream_shared: the waves of a workgroup walk the same blocks in
//    lockstep, each owning different rows, and stage the digit fragments
//    once per workgroup into an LDS ring with direct global-to-LDS loads;
//    one LDS-only barrier per stage.  Three to twelve waves by batch.
//  * k_rows_stream_valu (1 to 4 inputs, on request): the same digits on the
//    vector ALU instead of the matrix cores, v_dot4_i32_i8 adding four
//    byte products per instruction, with the inputs' digits resident in LDS
//    for the whole launch.  It computes the same words; measured over
//    stacked 4096-column matrices it streams a little slower than the
//    matrix-core kernel at 1 and 2 inputs and much slower from 4 on, so the
//    library takes it only when asked to (fpi8_matrix_rows_set_path).
//
// A launch whose inputs hold a word beyond three digits takes an exact
// 64-bit loop instead, so the result is the page's for every input.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/fpi8.h"
#include "fpi8_device.h"
#include "fpi8_internal.h"

namespace fpi8 {

namespace {

// The exact path (a cold path; written as one output at a time, so that its
// registers stay below the streaming loop's): y of every row and run this
// lane holds in the tile, from 64-bit sums over the packed bytes.  Inlined:
// a call would give the kernel a stack, whose scratch setup cost about 5%
// of a launch over the stacked 4096-column pool.
__device__ __forceinline__ void stream_exact(const RowsArgs &a, uint32_t ptile0, int mt_n, int bt_n,
                                                       int li, int lg) {
  const Seg &sg = a.seg[0];
  for (int mt = 0; mt < mt_n; mt++)
    for (int bt = 0; bt < bt_n; bt++)
      for (int j = 0; j < 4; j++) {
        const uint32_t row = (ptile0 + mt) * 16 + 4 * lg + j, b = bt * 16 + li;
        if (row >= sg.rows || b >= a.n_runs) continue;
        const uint8_t *P = sg.P + (uint64_t)(row / 16) * a.kblocks * 1024 + (row % 16) * 16;
        const int64_t *x = a.x_raw + (uint64_t)b * a.cols;
        int64_t s = 0;
        for (uint32_t k = 0; k < a.cols; k++) {
          const uint8_t wb = P[(uint64_t)(k / 64) * 1024 + ((k % 64) / 16) * 256 + k % 16];
          s = wadd(s, wmul((int64_t)wb - 128, x[k]));
        }
        a.y_raw[(uint64_t)b * sg.rows + row] = wmul(s, (int64_t)sg.S[row]) >> 24;
      }
}

// y[b][row] = (v * scale) >> 24 for the rows and runs this lane holds.
template <int MT, int BT>
__device__ __forceinline__ void stream_store(const RowsArgs &a, uint32_t ptile0, int li, int lg,
                                             const int64_t (&v)[MT][BT][4], const uint32_t (&sc)[MT][4]) {
  const uint32_t rows = a.seg[0].rows;
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
    const uint32_t r0 = (ptile0 + mt) * 16 + 4 * lg;
#pragma unroll
    for (int bt = 0; bt < BT; bt++) {
      const uint32_t b = bt * 16 + li;
      if (b >= a.n_runs || r0 >= rows) continue;
      int64_t y[4];
#pragma unroll
      for (int j = 0; j < 4; j++) y[j] = wmul(v[mt][bt][j], (int64_t)sc[mt][j]) >> 24;
      int64_t *yp = a.y_raw + (uint64_t)b * rows + r0;
      if (r0 + 4 <= rows && (((uintptr_t)yp) & 15) == 0) {
        *reinterpret_cast<longlong2 *>(yp) = longlong2{y[0], y[1]};
        *reinterpret_cast<longlong2 *>(yp + 2) = longlong2{y[2], y[3]};
      } else {
#pragma unroll
        for (int j = 0; j < 4; j++)
          if (r0 + j < rows) yp[j] = y[j];
      }
    }
  }
}

template <int MT>
__device__ __forceinline__ void stream_scales(const RowsArgs &a, uint32_t ptile0, int lg, uint32_t (&sc)[MT][4]) {
  const Seg &sg = a.seg[0];
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const uint32_t r = (ptile0 + mt) * 16 + 4 * lg + j;
      sc[mt][j] = sg.S[r < sg.rows ? r : sg.rows - 1];
    }
}

__device__ __forceinline__ v4i flip_weights(v4i w) {
  const int f = (int)0x80808080u;
  w.x ^= f; w.y ^= f; w.z ^= f; w.w ^= f;
  return w;
}

}  // namespace

// Stages of CD blocks; the digits of a stage are 3 * BT * CD fragments, W
// waves issue FR / W of them each into LDS buffer s; the weights of the
// stage go to register slot s.  NB = P + 1 buffers (2 or 4): after the
// barrier of stage k every wave has finished stage k - 1, so stage k + P
// may refill its buffer.  kblocks / CD is a multiple of NB, so every tile
// starts at buffer 0.
template <int BT, int CD, int W>
struct StreamShared {
  static constexpr int FR = 3 * BT * CD;
  static constexpr int FW = FR / W;
  static_assert(FR % W == 0, "every wave stages the same number of fragments");
};

template <int I, int N>
__device__ __forceinline__ v4i *stream_ring() {
  __shared__ v4i buf[N];
  return buf;
}

template <int MT, int BT, int P, int CD, int W>
__global__ __launch_bounds__(64 * W) void k_rows_stream_shared(RowsArgs a) {
  using G_ = StreamShared<BT, CD, W>;
  constexpr int FR = G_::FR, FW = G_::FW, NB = P + 1;
  constexpr int NL = MT * CD + FW;  // loads per stage and wave
  static_assert(NB == 2 || NB == 4, "two or four ring buffers");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const Seg &sg = a.seg[0];
  const uint32_t nkb = a.kblocks, kbp = a.kp / 64, nbt = a.bp / 16, nch = nkb / CD;
  if (blockIdx.x >= a.ntiles) return;
  const uint32_t my = (a.ntiles - blockIdx.x + gridDim.x - 1) / gridDim.x;
  const uint32_t last_ptile = (sg.rows - 1) / 16;
  auto ptile_of = [&](uint32_t t) { return ((blockIdx.x + t * gridDim.x) * W + wave) * MT; };

  if (input_needs_exact(a)) {
    for (uint32_t t = 0; t < my; t++) stream_exact(a, ptile_of(t), MT, BT, li, lg);
    return;
  }

  v4i *ring[NB];
  ring[0] = stream_ring<0, FR * 64>();
  ring[1] = stream_ring<1, FR * 64>();
  if constexpr (NB == 4) {
    ring[2] = stream_ring<2, FR * 64>();
    ring[3] = stream_ring<3, FR * 64>();
  }
  // This wave stages fragments f = wave + W q of every stage: (limb l, run
  // tile bt, block c of the stage).
  const int8_t *dsrc[FW];
#pragma unroll
  for (int q = 0; q < FW; q++) {
    const int f = wave + W * q;
    const int l = f / (BT * CD), bt = (f / CD) % BT, c = f % CD;
    dsrc[q] = a.planes + ((((uint64_t)l * nbt + bt) * kbp + c) * 64 + lane) * 16;
  }
  v4i acc[MT][3][BT];
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int l = 0; l < 3; l++)
#pragma unroll
      for (int bt = 0; bt < BT; bt++) acc[mt][l][bt] = v4i{0, 0, 0, 0};
  v4i Wr[NB][MT][CD];

  uint32_t it = 0, ich = 0;
  auto issue = [&](int s) {
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t t = it < my ? it : my - 1;
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      uint32_t pt = ptile_of(t) + mt;
      pt = pt < last_ptile ? pt : last_ptile;
      const uint8_t *wp = sg.P + ((uint64_t)pt * nkb + (uint64_t)ich * CD) * 1024 + lane * 16;
#pragma unroll
      for (int c = 0; c < CD; c++)
        Wr[s][mt][c] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(wp + c * 1024));
    }
#pragma unroll
    for (int q = 0; q < FW; q++)
      __builtin_amdgcn_global_load_lds((const void *)(dsrc[q] + (uint64_t)ich * CD * 1024),
                                       (lds_void *)(ring[s] + (wave + W * q) * 64), 16, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (++ich == nch) {
      ich = 0;
      ++it;
    }
  };
  auto compute = [&](int s) {
    const v4i *buf = ring[s];
#pragma unroll
    for (int c = 0; c < CD; c++) {
      v4i w[MT];
#pragma unroll
      for (int mt = 0; mt < MT; mt++) w[mt] = flip_weights(Wr[s][mt][c]);
#pragma unroll
      for (int l = 0; l < 3; l++)
#pragma unroll
        for (int bt = 0; bt < BT; bt++) {
          const v4i Bv = buf[((l * BT + bt) * CD + c) * 64 + lane];
#pragma unroll
          for (int mt = 0; mt < MT; mt++)
            acc[mt][l][bt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[mt], Bv, acc[mt][l][bt], 0, 0, 0);
        }
    }
  };

#pragma unroll
  for (int s = 0; s < P; s++) issue(s);
  for (uint32_t t = 0; t < my; t++) {
    const uint32_t ptile0 = ptile_of(t);
    uint32_t sc[MT][4];
    stream_scales<MT>(a, ptile0, lg, sc);
    for (uint32_t ch = 0; ch < nch; ch += NB) {
#pragma unroll
      for (int s = 0; s < NB; s++) {
        wait_vm<(P - 1) * NL>();  // stage ch + s has landed (in-order completion)
        lds_barrier();            // ... for every wave, which has also finished stage ch + s - 1
        issue((s + P) % NB);
        compute(s);
      }
    }
    int64_t v[MT][BT][4];
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int bt = 0; bt < BT; bt++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          v[mt][bt][j] = (int64_t)acc[mt][0][bt][j] + ((int64_t)acc[mt][1][bt][j] << 8) +
                         ((int64_t)acc[mt][2][bt][j] << 16);
          acc[mt][0][bt][j] = 0;
          acc[mt][1][bt][j] = 0;
          acc[mt][2][bt][j] = 0;
        }
    stream_store<MT, BT>(a, ptile0, li, lg, v, sc);
  }
  wait_vm<0>();  // no staging load may still be landing in LDS when the workgroup ends
}

// The vector-ALU kernel.  Lane l = 16g + i holds row i of each 16-row tile
// and columns 16g .. 16g+15 of each 64-column block (the packed operand
// layout), so the 16 lanes of a group read the same 16 digit bytes from LDS
// (a broadcast).  Every workgroup first splits the NB inputs into their
// three signed byte digits, [input][digit][column] in LDS (zero past the
// last column), and notes a word beyond three digits, which sends every
// wave down the exact loop.  Each wave then walks its tiles as in
// k_rows_stream, a ring of P weight blocks ahead; per block it adds, for
// every tile, input and digit, four v_dot4_i32_i8 products into an i32 sum
// (exact: |sum| <= 2^14 * cols < 2^31).  At the end of a tile the four lane
// groups' sums of a row are added across lanes and recombined in i64.
template <int MT, int NB, int P>
__global__ __launch_bounds__(256) void k_rows_stream_valu(RowsArgs a) {
  extern __shared__ __align__(16) int8_t dig[];  // [NB][3][kblocks * 64]
  __shared__ uint32_t over;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const Seg &sg = a.seg[0];
  const uint32_t nkb = a.kblocks, K = nkb * 64, cols = a.cols;
  if (tid == 0) over = 0;
  __syncthreads();
  bool bad = false;
  for (uint32_t c = tid; c < NB * (K / 4); c += 256) {
    const uint32_t r = c / (K / 4), k4 = (c % (K / 4)) * 4;
    uint32_t w0 = 0, w1 = 0, w2 = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      if (k4 + j >= cols) break;
      int8_t d0, d1, d2;
      bad |= !digits3(a.x_raw[(uint64_t)r * cols + k4 + j], d0, d1, d2);
      w0 |= (uint32_t)(uint8_t)d0 << (8 * j);
      w1 |= (uint32_t)(uint8_t)d1 << (8 * j);
      w2 |= (uint32_t)(uint8_t)d2 << (8 * j);
    }
    *reinterpret_cast<uint32_t *>(dig + ((uint64_t)r * 3 + 0) * K + k4) = w0;
    *reinterpret_cast<uint32_t *>(dig + ((uint64_t)r * 3 + 1) * K + k4) = w1;
    *reinterpret_cast<uint32_t *>(dig + ((uint64_t)r * 3 + 2) * K + k4) = w2;
  }
  if (bad) atomicOr(&over, 1u);
  __syncthreads();

  const uint32_t G = gridDim.x * 4, gw = blockIdx.x * 4 + wave;
  if (gw >= a.ntiles) return;
  const uint32_t my = (a.ntiles - gw + G - 1) / G;  // tiles of this wave
  const uint32_t last_ptile = (sg.rows - 1) / 16;
  if (over) {
    for (uint32_t t = 0; t < my; t++) stream_exact(a, (gw + t * G) * MT, MT, 1, li, lg);
    return;
  }

  int acc[MT][NB][3];
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int r = 0; r < NB; r++) acc[mt][r][0] = acc[mt][r][1] = acc[mt][r][2] = 0;
  v4i Wr[P][MT];
  uint32_t it = 0, ikb = 0;
  auto issue = [&](int s) {
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t t = it < my ? it : my - 1;
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      uint32_t pt = (gw + t * G) * MT + mt;
      pt = pt < last_ptile ? pt : last_ptile;
      Wr[s][mt] = __builtin_nontemporal_load(
          reinterpret_cast<const v4i *>(sg.P + ((uint64_t)pt * nkb + ikb) * 1024 + lane * 16));
    }
    __builtin_amdgcn_sched_barrier(0);
    if (++ikb == nkb) {
      ikb = 0;
      ++it;
    }
  };
  auto compute = [&](int s, uint32_t kb) {
    v4i w[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) w[mt] = flip_weights(Wr[s][mt]);
#pragma unroll
    for (int r = 0; r < NB; r++)
#pragma unroll
      for (int d = 0; d < 3; d++) {
        const v4i dv = *reinterpret_cast<const v4i *>(dig + ((uint64_t)r * 3 + d) * K + kb * 64 + lg * 16);
#pragma unroll
        for (int mt = 0; mt < MT; mt++) {
          int c = acc[mt][r][d];
          c = __builtin_amdgcn_sdot4(w[mt].x, dv.x, c, false);
          c = __builtin_amdgcn_sdot4(w[mt].y, dv.y, c, false);
          c = __builtin_amdgcn_sdot4(w[mt].z, dv.z, c, false);
          c = __builtin_amdgcn_sdot4(w[mt].w, dv.w, c, false);
          acc[mt][r][d] = c;
        }
      }
  };

#pragma unroll
  for (int s = 0; s < P; s++) issue(s);
  for (uint32_t t = 0; t < my; t++) {
    const uint32_t ptile0 = (gw + t * G) * MT;
    for (uint32_t kb = 0; kb < nkb; kb += P) {
#pragma unroll
      for (int s = 0; s < P; s++) {
        compute(s, kb + s);
        issue(s);
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      const uint32_t row = (ptile0 + mt) * 16 + li;
      const uint32_t sc = sg.S[row < sg.rows ? row : sg.rows - 1];
#pragma unroll
      for (int r = 0; r < NB; r++) {
        int s3[3];
#pragma unroll
        for (int d = 0; d < 3; d++) {
          int v = acc[mt][r][d];
          v += __shfl_xor(v, 16);
          v += __shfl_xor(v, 32);
          s3[d] = v;
          acc[mt][r][d] = 0;
        }
        const int64_t v = (int64_t)s3[0] + ((int64_t)s3[1] << 8) + ((int64_t)s3[2] << 16);
        if (lg == 0 && row < sg.rows) a.y_raw[(uint64_t)r * sg.rows + row] = wmul(v, (int64_t)sc) >> 24;
      }
    }
  }
  wait_vm<0>();  // the ring's last (unused) loads land before the wave ends
}

// ---------------------------------------------------------------------------

namespace {

int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

template <int MT, int BT, int P, int CD, int W>
int launch_shr(RowsArgs a, hipStream_t s) {
  a.ntiles = (a.seg[0].rows + W * 16 * MT - 1) / (W * 16 * MT);
  const uint32_t wgs = std::min<uint32_t>(a.ntiles, (uint32_t)cu_count());
  hipLaunchKernelGGL((k_rows_stream_shared<MT, BT, P, CD, W>), dim3(wgs), dim3(64 * W), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : FPI8_ERR_HIP;
}

}  // namespace

uint32_t stream_min_rows() { return (uint32_t)cu_count() * 256u; }

namespace {

template <int NB>
int launch_valu(RowsArgs a, hipStream_t s) {
  constexpr int MT = 4, P = 4;
  const size_t lds = (size_t)NB * 3 * a.kblocks * 64;
  if (hipFuncSetAttribute((const void *)k_rows_stream_valu<MT, NB, P>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStreamValuLds) != hipSuccess)
    return FPI8_ERR_HIP;
  a.ntiles = (a.seg[0].rows + 16 * MT - 1) / (16 * MT);
  const uint32_t wgs = std::min<uint32_t>((a.ntiles + 3) / 4, (uint32_t)cu_count());
  hipLaunchKernelGGL((k_rows_stream_valu<MT, NB, P>), dim3(wgs), dim3(256), lds, s, a);
  return hipGetLastError() == hipSuccess ? 0 : FPI8_ERR_HIP;
}

}  // namespace

bool stream_valu_fits(uint32_t kblocks, uint32_t n_runs) {
  return n_runs >= 1 && n_runs <= 4 && kblocks % 4 == 0 &&
         (uint64_t)n_runs * 3 * kblocks * 64 <= kStreamValuLds;
}

int launch_rows_stream_valu(const RowsArgs &a, void *stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.nseg != 1 || !a.seg[0].P || !a.x_raw || !a.y_raw || !stream_valu_fits(a.kblocks, a.n_runs))
    return FPI8_ERR_ARGUMENT;
  switch (a.n_runs) {
    case 1: return launch_valu<1>(a, s);
    case 2: return launch_valu<2>(a, s);
    case 3: return launch_valu<3>(a, s);
    default: return launch_valu<4>(a, s);
  }
}

// The launch shapes by batch, measured on MI355X over a pool of 48
// 4096-column matrices, all staging one block of digit fragments per stage:
// up to 16 runs, 3 waves x 64 rows (each wave stages one digit plane);
// 17-32 runs, 6 waves x 64 rows; 33-64 runs, 12 waves x 32 rows; 65-128
// runs, 12 waves x 16 rows with two ring buffers.  More waves than the four
// SIMDs keep more weight loads in flight; one block per stage keeps the
// waves closest together.
int launch_rows_stream(const RowsArgs &a, void *stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.nseg != 1 || !a.seg[0].P || a.compact || a.n_runs == 0 || a.n_runs > 128 ||
      a.kblocks % kStreamBlockMultiple != 0 || a.bp < (a.n_runs + 15) / 16 * 16)
    return FPI8_ERR_ARGUMENT;
  if (a.n_runs <= 16) return launch_shr<4, 1, 3, 1, 3>(a, s);
  if (a.n_runs <= 32) {
    if (a.bp < 32) return FPI8_ERR_ARGUMENT;
    return launch_shr<4, 2, 3, 1, 6>(a, s);
  }
  if (a.n_runs <= 64) {
    if (a.bp < 64) return FPI8_ERR_ARGUMENT;
    return launch_shr<2, 4, 1, 1, 12>(a, s);
  }
  if (a.bp < 128) return FPI8_ERR_ARGUMENT;
  return launch_shr<1, 8, 1, 1, 12>(a, s);
}

}  // namespace fpi8
