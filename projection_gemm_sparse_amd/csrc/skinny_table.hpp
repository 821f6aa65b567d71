// skinny_table.hpp -- compiled configurations of the vector-ALU kernel, as
// kernel addresses (host side of the k_skinny_*.hip units).  Each unit calls
// the table of its own family, so every instantiation is emitted once.
#pragma once

#include "skinny.hpp"

namespace fpk_detail {

template <int MT, int CJ, bool BF16, int VAR>
const void* skinny_rw(int rw) {
  switch (rw) {
    case 1: return reinterpret_cast<const void*>(&fp::skinny_kernel<MT, 1, CJ, BF16, VAR>);
    case 2: return reinterpret_cast<const void*>(&fp::skinny_kernel<MT, 2, CJ, BF16, VAR>);
    case 3: return reinterpret_cast<const void*>(&fp::skinny_kernel<MT, 3, CJ, BF16, VAR>);
    case 4: return reinterpret_cast<const void*>(&fp::skinny_kernel<MT, 4, CJ, BF16, VAR>);
    case 5: return reinterpret_cast<const void*>(&fp::skinny_kernel<MT, 5, CJ, BF16, VAR>);
    case 6: return reinterpret_cast<const void*>(&fp::skinny_kernel<MT, 6, CJ, BF16, VAR>);
    case 7: return reinterpret_cast<const void*>(&fp::skinny_kernel<MT, 7, CJ, BF16, VAR>);
    case 8: return reinterpret_cast<const void*>(&fp::skinny_kernel<MT, 8, CJ, BF16, VAR>);
    default: return nullptr;
  }
}

// Long per-lane chunk runs (a wave covering a whole row): one or two rows
// per wave.
template <int MT, int CJ, bool BF16>
const void* skinny_rw_long(int rw) {
  switch (rw) {
    case 1: return reinterpret_cast<const void*>(&fp::skinny_kernel<MT, 1, CJ, BF16>);
    case 2: return reinterpret_cast<const void*>(&fp::skinny_kernel<MT, 2, CJ, BF16>);
    default: return nullptr;
  }
}

// Plain projections: one or two chunks per lane at any RW; long runs
// (4..12 chunks) for at most two tokens.
template <int MT, bool BF16>
const void* skinny_plain_cj(int cj, int rw) {
  switch (cj) {
    case 1: return skinny_rw<MT, 1, BF16, fp::kVarPlain>(rw);
    case 2: return skinny_rw<MT, 2, BF16, fp::kVarPlain>(rw);
    default: break;
  }
  if constexpr (MT <= 2) {
    switch (cj) {
      case 4: return skinny_rw_long<MT, 4, BF16>(rw);
      case 5: return skinny_rw_long<MT, 5, BF16>(rw);
      case 6: return skinny_rw_long<MT, 6, BF16>(rw);
      case 8: return skinny_rw_long<MT, 8, BF16>(rw);
      case 10: return skinny_rw_long<MT, 10, BF16>(rw);
      case 12: return skinny_rw_long<MT, 12, BF16>(rw);
      default: break;
    }
  }
  return nullptr;
}

template <bool BF16>
const void* skinny_plain(int mt, int cj, int rw) {
  switch (mt) {
    case 1: return skinny_plain_cj<1, BF16>(cj, rw);
    case 2: return skinny_plain_cj<2, BF16>(cj, rw);
    case 4: return skinny_plain_cj<4, BF16>(cj, rw);
    case 8: return skinny_plain_cj<8, BF16>(cj, rw);
    default: return nullptr;
  }
}

// Gate/up launches (PAIRS): bf16, an even number of rows per wave, one or
// two chunks per lane.
template <int MT, int CJ>
const void* skinny_pairs_rw(int rw) {
  switch (rw) {
    case 2: return reinterpret_cast<const void*>(&fp::skinny_kernel<MT, 2, CJ, true, fp::kVarPairs>);
    case 4: return reinterpret_cast<const void*>(&fp::skinny_kernel<MT, 4, CJ, true, fp::kVarPairs>);
    case 6: return reinterpret_cast<const void*>(&fp::skinny_kernel<MT, 6, CJ, true, fp::kVarPairs>);
    case 8: return reinterpret_cast<const void*>(&fp::skinny_kernel<MT, 8, CJ, true, fp::kVarPairs>);
    default: return nullptr;
  }
}

template <int MT>
const void* skinny_pairs_cj(int cj, int rw) {
  switch (cj) {
    case 1: return skinny_pairs_rw<MT, 1>(rw);
    case 2: return skinny_pairs_rw<MT, 2>(rw);
    default: return nullptr;
  }
}

// fp32 outputs from bf16 operands (router logits): up to 16 tokens, one or
// two chunks per lane, at most 64 outputs per lane.
template <int MT, int CJ>
const void* skinny_f32out_rw(int rw) {
  switch (rw) {
    case 1: return reinterpret_cast<const void*>(&fp::skinny_kernel<MT, 1, CJ, true, fp::kVarF32Out>);
    case 2: return reinterpret_cast<const void*>(&fp::skinny_kernel<MT, 2, CJ, true, fp::kVarF32Out>);
    case 4: return reinterpret_cast<const void*>(&fp::skinny_kernel<MT, 4, CJ, true, fp::kVarF32Out>);
    default: break;
  }
  if constexpr (MT <= 8) {
    if (rw == 8) return reinterpret_cast<const void*>(&fp::skinny_kernel<MT, 8, CJ, true, fp::kVarF32Out>);
  }
  return nullptr;
}

template <int MT>
const void* skinny_f32out_cj(int cj, int rw) {
  switch (cj) {
    case 1: return skinny_f32out_rw<MT, 1>(rw);
    case 2: return skinny_f32out_rw<MT, 2>(rw);
    default: return nullptr;
  }
}

// Block-scaled weights: up to 8 tokens, one or two units per lane.
template <int VAR, int MT>
const void* skinny_mx_cj(int cj, int rw) {
  switch (cj) {
    case 1: return skinny_rw<MT, 1, true, VAR>(rw);
    case 2: return skinny_rw<MT, 2, true, VAR>(rw);
    default: return nullptr;
  }
}

template <int VAR>
const void* skinny_mx(int mt, int cj, int rw) {
  switch (mt) {
    case 1: return skinny_mx_cj<VAR, 1>(cj, rw);
    case 2: return skinny_mx_cj<VAR, 2>(cj, rw);
    case 4: return skinny_mx_cj<VAR, 4>(cj, rw);
    case 8: return skinny_mx_cj<VAR, 8>(cj, rw);
    default: return nullptr;
  }
}

}  // namespace fpk_detail
