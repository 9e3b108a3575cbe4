// Byte geometry of one INT2 page-head and one BF16 page-head (the layout
// defined in include/oscar.h), shared by the kernels.
#pragma once

namespace oscar_dev {

template <int D>
struct Geo {
  static constexpr int NG = D / 32;    // channel groups
  static constexpr int NCB = D / 16;   // 16-channel blocks
  static constexpr int NKB = D / 32;   // 32-wide reduction blocks
  static constexpr int NW = D / 64;    // code words per lane per page
  static constexpr int HEAD_BYTES = 12 * D;
  static constexpr int KC = 0;
  static constexpr int VC = 4 * D;
  static constexpr int KS = 8 * D;
  static constexpr int KZ = 8 * D + 32 * NG;
  static constexpr int VS = 8 * D + 64 * NG;
  static constexpr int VZ = 8 * D + 96 * NG;
  static constexpr int BF16_HEAD_ELEMS = 32 * D;  // K [16][D] then V [D][16]
};

// INT4 page-head (the 16-level variant): K codes [16 slots][D/2] bytes, V
// codes [16][D/2] (channel 2i in the low nibble of byte i), then f16 K
// scales, K zeros, V scales, V zeros, each [16 slots][NG].
template <int D>
struct Geo4 {
  static constexpr int NG = D / 32;
  static constexpr int HEAD_BYTES = 20 * D;
  static constexpr int KC = 0;
  static constexpr int VC = 8 * D;
  static constexpr int KS = 16 * D;
  static constexpr int KZ = 16 * D + 32 * NG;
  static constexpr int VS = 16 * D + 64 * NG;
  static constexpr int VZ = 16 * D + 96 * NG;
};

// The quantized page-head of a code width: Geo (INT2) or Geo4 (INT4).
template <int D, int BITS>
struct QLayout;
template <int D>
struct QLayout<D, 2> : Geo<D> {};
template <int D>
struct QLayout<D, 4> : Geo4<D> {};

}  // namespace oscar_dev
