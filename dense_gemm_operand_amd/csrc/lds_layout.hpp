// LDS tile layout: K-contiguous rows, a pad after every row, and a block permutation of
// the rows.
//
// Rows. Every operand tile lives in LDS as one row per M (or N) index holding its BK
// K-consecutive elements, whatever the operand's global layout (Triton PR 5223, "PR
// description", item 1: the shared order is swapped for non-KContig tensors so that LDS
// reads stay coalesced). Matrix-core fragments are then one 16-byte read per lane.
//
// Pad. Each row is followed by `pad` bytes (a multiple of 16 so that every 16-byte
// store and load stays aligned; Triton PR 5223 item 3 aligns shared addresses to the
// vector written). With a 128-byte row and a 16-byte pad, consecutive rows start in
// consecutive 16-byte bank groups, so the eight lanes of one 128-bit access phase that
// read eight consecutive rows hit eight different bank groups.
//
// Permutation. Within blocks of `block` rows, LDS row I holds logical row
// fwd(I) = S*(I mod S') + I div S' with S' = block / S, and logical row I' is found at LDS
// row inv(I') = S'*(I' mod S) + I' div S (rocm-libraries PR 2487, "Add support for
// permuting perpDim": forward map for the global-read side, inverse for the local-read
// side). For an operand that is transposed in registers, one lane owns eight consecutive
// logical rows (one 16-byte global vector along M or N), so the eight lanes of one
// write phase store rows 8v + j for eight consecutive v. With block = 64 and S = 8, inv
// sends those rows to eight consecutive LDS rows, i.e. eight different bank groups; the
// readers walk LDS rows in order and the epilogue maps LDS row I back to logical fwd(I).
#pragma once

namespace dg {

struct RowPerm {
  int block;   // rows per permutation block (1 = identity)
  int stride;  // S; must divide block

  __host__ __device__ constexpr bool valid() const {
    return block >= 1 && stride >= 1 && stride <= block && block % stride == 0;
  }
  // LDS row -> logical row.
  __host__ __device__ constexpr int fwd(int I) const {
    const int sp = block / stride;
    const int b = I / block, i = I - b * block;
    return b * block + stride * (i % sp) + i / sp;
  }
  // logical row -> LDS row.
  __host__ __device__ constexpr int inv(int Ip) const {
    const int sp = block / stride;
    const int b = Ip / block, i = Ip - b * block;
    return b * block + sp * (i % stride) + i / stride;
  }
};

}  // namespace dg
