// Fast bf16 WBMM forward for w = 14, NCHW, square images of 28x28 or 56x56, table input, bf16
// output, no 3x3 mix. With bf16 operands the window contraction needs little matrix time
// (v_mfma_f32_16x16x32_bf16 does 16x16x32 per instruction), so this kernel is built to move the
// map through HBM once each way at full rate with as few instructions per byte as possible:
//   * a unit = 64 windows of one channel (4 wave-units of 16 windows, whole images); three
//     persistent workgroups per CU each walk a run of consecutive units (one channel, so the
//     table is staged once), every wave keeping the next unit's pixels in flight while it
//     contracts and stores the current one;
//   * loads and stores move 112-pixel chunks (8 window rows of 7 pixel pairs, 56 lanes) that are
//     contiguous in the map, so every per-chunk address is a per-lane base plus an immediate;
//   * a wave-unit sits in LDS image-major with every 14-pixel window row padded to 16 (zeros),
//     so K = 224 is 7 steps of 32 and each MFMA operand (8 pixels of a window row) is one aligned
//     16-byte read; 16-byte gaps between the four row blocks put the 16 windows of a step on
//     distinct bank quads;
//   * M_c is never formed: the table is reversed with its rows padded to a pitch of 32, and 8
//     copies shifted by 0..7 make any 8-entry run of a row one aligned 16-byte read; with pitch
//     32 the copy a pixel row needs is the same at every K step, so each step's read is again
//     base + immediate [gecl.asia reading notes, "Core Idea"; the notes' "Limitation" and
//     "Takeaway" name such a kernel as future work];
//   * the contraction is computed transposed (X^T M^T: windows are MFMA rows, output pixels are
//     columns), which makes the output positions of a lane base + immediate as well; results are
//     rounded to bf16 (RNE, v_cvt_pk_bf16_f32) into LDS over the inputs, then stored by chunks.
#include "wbmm_device.hpp"
#include "wbmm_launch.hpp"

#include <type_traits>

namespace wbmm {
namespace {

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

struct BfArgs {
  int B, C;
  int groups;  // units per channel: ceil(B / images per unit)
  const uint16_t* x;
  const uint16_t* T;
  uint16_t* y;
  uint16_t* z;  // optional copy of the output (the pre-mix map equals y without a mix)
};

template <int IW_>
struct BfShape {
  static constexpr int WS = 14, IH = IW_, IW = IW_;
  static constexpr int D = WS * WS;
  static constexpr int RT = (D + 15) / 16;        // 16-pixel output tiles
  static constexpr int L1 = 2 * WS - 1;
  static constexpr int NWX = IW / WS, NWIN = NWX * NWX;
  static constexpr int IPW = 16 / NWIN;           // images per wave-unit
  static constexpr int PLANE = IH * IW;
  static constexpr int SEG = 16;                  // LDS pixels per window row (14 + 2 zeros)
  static constexpr int HP = SEG * NWX;            // LDS pitch of an image row
  // a wave-unit is four LDS blocks: the four window-row bands of one 56x56 image, or four
  // 28x28 images
  static constexpr int BROWS = IW == 56 ? WS : IH;
  static constexpr int BLK = BROWS * HP;
  static constexpr int CHUNK = 112;               // pixels per load/store chunk
  static constexpr int RPC = CHUNK / IW;          // image rows per chunk
  static constexpr int CPB = BROWS * IW / CHUNK;  // chunks per block
  static constexpr int NCH = 4 * CPB;             // chunks per wave-unit
  // quads (16 bytes) of gap before block b: with these the 16 windows of a wave-unit start on
  // 16 distinct bank quads
  static constexpr int gap(int b) { return (b & 1) + (IW == 56 ? 8 : 4) * (b >> 1); }
  static constexpr int bstart(int b) { return b * BLK + 8 * gap(b); }
  static constexpr int RSZ = bstart(3) + BLK;     // bf16 per wave-unit region
  static constexpr int TP = 32;                   // padded table row pitch
  static constexpr int PT = L1 * TP;              // padded table entries
  static constexpr int CS = 912;                  // bf16 per shifted copy (copy r starts r*CS)
  static_assert(IW == 28 || IW == 56, "shape");
  static_assert(BROWS * IW % CHUNK == 0 && 8 % NWX == 0, "chunks");
  static_assert(CS % 8 == 0 && CS >= PT + 16, "copies");
  static_assert((RSZ * 2) % 16 == 0 && (BLK * 2) % 256 == 0, "region alignment");
};

template <class S>
constexpr int bf_lds_bytes() { return (8 * S::CS + 4 * S::RSZ) * 2; }

// LDS offset (bf16) of the first pixel of window m (0..15) of a wave-unit region: windows are
// numbered block-major, then window row, then window column.
template <class S>
__device__ __forceinline__ int wstart(int m) {
  const int b = m >> 2, k = m & 3;
  return b * S::BLK + 8 * ((b & 1) + (S::IW == 56 ? 8 : 4) * (b >> 1)) +
         (k / S::NWX) * S::WS * S::HP + S::SEG * (k % S::NWX);
}

// Offset of window 4g + r relative to window 4g (the same for every g).
template <class S>
constexpr int woff(int r) { return (r / S::NWX) * S::WS * S::HP + S::SEG * (r % S::NWX); }

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Where unit u's data live: channel c, first image, images in the unit.
struct UnitPos {
  int c, img0, nimg;
};
__device__ __forceinline__ UnitPos unit_pos(const BfArgs& a, int u, int ipu) {
  UnitPos p;
  p.c = u / a.groups;
  p.img0 = (u - p.c * a.groups) * ipu;
  p.nimg = min(a.B - p.img0, ipu);
  return p;
}

// Element offset of block b of this wave's share of unit p (its image plane, plus the band
// offset for 56x56 images); images past the batch are clamped to its last image.
template <class S>
__device__ __forceinline__ size_t block_base(const BfArgs& a, const UnitPos& p, int wave, int b) {
  const int im = wave * S::IPW + (S::IW == 56 ? 0 : b);
  const int imc = im < p.nimg ? im : p.nimg - 1;
  return ((size_t)(p.img0 + imc) * a.C + p.c) * S::PLANE + (S::IW == 56 ? b * S::WS * S::IW : 0);
}

// Persistent: workgroup g walks the units [g*units/grid, (g+1)*units/grid) (a run of consecutive
// units shares a channel, so the table copies are rebuilt only when it changes); each wave owns
// one wave-unit region and has the next unit's pixels in flight while it contracts and stores
// the current one.
template <class S>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8)))
k_fwd_bf16(BfArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem_h[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  uint16_t* copies = smem_h;  // [8][CS]
  uint16_t* R = smem_h + 8 * S::CS + wave * S::RSZ;
  uint32_t* R32 = (uint32_t*)R;
  const int units = a.C * a.groups;
  const int u0 = (int)((long long)blockIdx.x * units / gridDim.x);
  const int u1 = (int)((long long)(blockIdx.x + 1) * units / gridDim.x);
  if (u0 >= u1) return;  // uniform over the workgroup
  constexpr int IPU = 4 * S::IPW;  // images per unit

  // the two padding pixels of every window row (K slots 14, 15) stay zero: neither the pixel
  // commits nor the output writes touch them
  for (int e = lane; e < 4 * S::BROWS * S::NWX; e += 64) {
    const int b = e / (S::BROWS * S::NWX), rr = e % (S::BROWS * S::NWX);
    R32[(b * S::BLK + 8 * S::gap(b) + (rr / S::NWX) * S::HP + S::SEG * (rr % S::NWX) + S::WS) >> 1] = 0u;
  }

  // chunk lanes: 56 lanes = 8 window rows x 7 pixel pairs; lanes 56..63 repeat lane 55 (same
  // load, same LDS word, same store: harmless duplicates, no divergent branches)
  const int lc = lane < 56 ? lane : 55;
  const int wr = lc / 7, q7 = lc - 7 * (lc / 7);
  const int lds_lane = (wr / S::NWX) * S::HP + S::SEG * (wr % S::NWX) + 2 * q7;  // bf16
  const int glb_lane = 2 * lc;                                                  // pixels

  uint32_t pv[S::NCH];
  auto issue = [&](const UnitPos& p) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t* src = (const uint32_t*)(a.x + block_base<S>(a, p, wave, b) + glb_lane);
#pragma unroll
      for (int jj = 0; jj < S::CPB; ++jj) pv[b * S::CPB + jj] = src[jj * S::CHUNK / 2];
    }
  };

  // per-lane MFMA operand bases (bf16 offsets), the same for every unit
  const int m = lane & 15, gq = lane >> 4;
  const int kq = (gq >> 1), kh = gq & 1;        // K block: window row 2s + kq, pixels 8kh..
  const int xb = wstart<S>(m) + kq * S::HP + 8 * kh;
  int ab[S::RT], ob[S::RT];
#pragma unroll
  for (int t = 0; t < S::RT; ++t) {
    // output pixel i of the tile column (lanes past the last pixel repeat it: same value, same
    // address)
    const int i = min(t * 16 + m, S::D - 1);
    const int yi = i / S::WS, xi = i - S::WS * (i / S::WS);
    // reversed padded table: M[i][(yj, xj)] = Rv[bi + 32 yj + xj], Rv[q] = Tpad[PT-1-q]
    const int bi = S::PT - 1 - (S::WS - 1) * S::TP - (S::WS - 1) - S::TP * yi - xi;
    const int r = (-bi) & 7;  // copy whose runs starting at bi (mod 8) are 16-byte aligned
    ab[t] = r * S::CS + bi + r + S::TP * kq + 8 * kh;
    ob[t] = wstart<S>(4 * gq) + yi * S::HP + xi;
  }

  UnitPos cur = unit_pos(a, u0, IPU);
  issue(cur);
  int table_c = -1;
  for (int u = u0; u < u1; ++u) {
    if (cur.c != table_c) {  // uniform: rebuild the 8 reversed, shifted, padded table copies
      constexpr int NQ = (S::CS + kThreads - 1) / kThreads;
      uint16_t tv[NQ];
      const uint16_t* Tc = a.T + (size_t)cur.c * S::L1 * S::L1;
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const int q = threadIdx.x + j * kThreads;
        const int p = S::PT - 1 - q;  // padded table index
        const bool in = p >= 0 && (p & (S::TP - 1)) < S::L1;
        const int ti = in ? (p / S::TP) * S::L1 + (p & (S::TP - 1)) : 0;
        tv[j] = Tc[ti];
        if (!in) tv[j] = 0;
      }
      __syncthreads();  // every wave is done with the previous copies
      // copy r holds Rv[q] at q + r; entries q >= CS - 7 lie past every read
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const int q = threadIdx.x + j * kThreads;
        if ((j + 1) * kThreads <= S::CS - 7 || q < S::CS - 7) {
#pragma unroll
          for (int r = 0; r < 8; ++r) copies[r * S::CS + q + r] = tv[j];
        }
      }
      __syncthreads();
      table_c = cur.c;
    }
    // commit the pixels to the region
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int jj = 0; jj < S::CPB; ++jj)
        R32[(S::bstart(b) + jj * S::RPC * S::HP + lds_lane) >> 1] = pv[b * S::CPB + jj];
    wave_sync();
    // the next unit's pixels are in flight from here on (the last unit re-reads itself, so the
    // loads need no branch)
    const UnitPos pos = cur;
    cur = unit_pos(a, u + 1 < u1 ? u + 1 : u, IPU);
    issue(cur);

    // out^T[window 4gq + r][pixel 16t + m] = sum_k X^T[window][k] M^T[k][pixel], k over 7 steps
    // of 32: lane group gq takes K block 4s + gq = window row 2s + kq, pixels 8kh .. 8kh + 7
    u32x4 xv[7];
#pragma unroll
    for (int s = 0; s < 7; ++s) xv[s] = *(const u32x4*)(R + xb + 2 * s * S::HP);
    auto half = [&](auto t0c, auto ntc) {
      constexpr int T0 = decltype(t0c)::value, NT = decltype(ntc)::value;
      // (s, t) steps, t fastest; table reads PD steps ahead
      constexpr int N = 7 * NT, PD = S::IW == 56 ? 3 : 2;
      v4f acc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
      u32x4 mv[PD + 1];
#pragma unroll
      for (int k = 0; k < PD; ++k)
        mv[k] = *(const u32x4*)(copies + ab[T0 + k % NT] + 2 * S::TP * (k / NT));
#pragma unroll
      for (int k = 0; k < N; ++k) {
        if (k + PD < N) {
          const int kn = k + PD;
          mv[kn % (PD + 1)] = *(const u32x4*)(copies + ab[T0 + kn % NT] + 2 * S::TP * (kn / NT));
        }
        acc[k % NT] = mfma_bf16(xv[k / NT], mv[k % (PD + 1)], acc[k % NT]);
        // keep this order: the scheduler otherwise trades the read-ahead for registers
        __builtin_amdgcn_sched_barrier(0);
      }
      // every lane's pixel reads are complete (the MFMAs consumed them), so the results may
      // overwrite the region
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const v2bf h = __builtin_convertvector((v2f{acc[t][r], acc[t][r + 1]}), v2bf);
          const uint32_t hw = __builtin_bit_cast(uint32_t, h);
          R[ob[T0 + t] + woff<S>(r)] = (uint16_t)hw;
          R[ob[T0 + t] + woff<S>(r + 1)] = (uint16_t)(hw >> 16);
        }
    };
    constexpr int H0 = (S::RT + 1) / 2;
    half(std::integral_constant<int, 0>{}, std::integral_constant<int, H0>{});
    half(std::integral_constant<int, H0>{}, std::integral_constant<int, S::RT - H0>{});
    wave_sync();
    // store the region by chunks (images past the batch are skipped: a uniform branch)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (wave * S::IPW + (S::IW == 56 ? 0 : b) >= pos.nimg) continue;
      uint32_t w[S::CPB];
#pragma unroll
      for (int jj = 0; jj < S::CPB; ++jj)
        w[jj] = R32[(S::bstart(b) + jj * S::RPC * S::HP + lds_lane) >> 1];
      const size_t o = block_base<S>(a, pos, wave, b) + glb_lane;
      uint32_t* yd = (uint32_t*)(a.y + o);
#pragma unroll
      for (int jj = 0; jj < S::CPB; ++jj) yd[jj * S::CHUNK / 2] = w[jj];
      if (a.z) {
        uint32_t* zd = (uint32_t*)(a.z + o);
#pragma unroll
        for (int jj = 0; jj < S::CPB; ++jj) zd[jj * S::CHUNK / 2] = w[jj];
      }
    }
    wave_sync();  // the next commit overwrites the region
  }
}

enum BfShapeId { BF_NONE, BF_28, BF_56 };

BfShapeId bf_shape(const FwdRequest& r) {
  if (r.layout != 0 || r.w != 14 || r.H != r.W) return BF_NONE;
  if (r.H == 28) return BF_28;
  if (r.H == 56) return BF_56;
  return BF_NONE;
}

constexpr int kLdsPerCu = 160 * 1024, kLdsGranule = 1280;
constexpr bool fits3(int bytes) {
  return (bytes + kLdsGranule - 1) / kLdsGranule * kLdsGranule * 3 <= kLdsPerCu;
}
static_assert(fits3(bf_lds_bytes<BfShape<28>>()) && fits3(bf_lds_bytes<BfShape<56>>()),
              "three workgroups per CU");

template <class S>
hipError_t launch_bf(const FwdRequest& r, hipStream_t st) {
  BfArgs a{};
  a.B = r.B;
  a.C = r.C;
  a.groups = (r.B + 4 * S::IPW - 1) / (4 * S::IPW);
  a.x = (const uint16_t*)r.x;
  a.T = (const uint16_t*)r.T;
  a.y = (uint16_t*)r.y;
  a.z = (uint16_t*)r.zsave;
  const int lds = bf_lds_bytes<S>();
  hipError_t e = hipFuncSetAttribute((const void*)k_fwd_bf16<S>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const int units = a.C * a.groups;
  const int grid = units < 3 * cus ? units : 3 * cus;  // three resident workgroups per CU
  mark_main_kernel(st, true);
  hipLaunchKernelGGL(k_fwd_bf16<S>, dim3(grid), dim3(kThreads), lds, st, a);
  e = hipGetLastError();
  mark_main_kernel(st, false);
  return e;
}

}  // namespace

bool fast_bf16_forward_ok(const FwdRequest& r) {
  // unit indices (C * groups) are ints
  return r.in_bf16 && r.out_bf16 && r.T && !r.M && !r.mixw && r.B > 0 && r.C > 0 &&
         (long long)r.C * ((r.B + 3) / 4 + 1) < ((long long)1 << 31) && bf_shape(r) != BF_NONE;
}

hipError_t launch_forward_fast_bf16(const FwdRequest& r, hipStream_t st) {
  switch (bf_shape(r)) {
    case BF_28: return launch_bf<BfShape<28>>(r, st);
    case BF_56: return launch_bf<BfShape<56>>(r, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wbmm
