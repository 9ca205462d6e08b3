// Block layout of the packed cache, shared by the kernels and the host API
// (plain constexpr: usable on both sides).
//
// A block holds the 16 slots of one (page, KV head): 1024 bytes of code words
// (64 records of 16 B), then one metadata record of 32 B per (group of G
// channels, slot quad): 128 * (128 / G) bytes, so 1536, 1280 or 1152 bytes
// for G = 32, 64, 128.  3- and 4-bit codes keep their low two bits in the
// code words and the rest in a plane per widened tensor after the metadata,
// the keys' plane first: 4 bits, 512 bytes (64 records of 8 B: record r at
// 8 r, words at the bits of the two K or V words of record r); 3 bits, 256
// bytes (64 records of 4 B, one word per record: a key's high bit at its low
// bits' position plus the word index, a value's at bit 8 (slot % 4) + channel
// / 16).
#pragma once

namespace kvq {

constexpr int kCodeBytes = 1024;    // 64 records x 16 B of K/V code words
constexpr int kMetaRecordBytes = 32;
constexpr int kBlockBytes = 1536;   // the largest 2-bit block (G = 32)

constexpr int meta_bytes(int gsize) { return 4 * kMetaRecordBytes * (128 / gsize); }
constexpr int plane_bytes(int bits) { return bits == 2 ? 0 : (bits == 3 ? 256 : 512); }
constexpr int k_hi_plane(int gsize) { return kCodeBytes + meta_bytes(gsize); }
constexpr int v_hi_plane(int kbits, int gsize) { return k_hi_plane(gsize) + plane_bytes(kbits); }
constexpr int block_bytes(int kbits, int vbits, int gsize) { return v_hi_plane(kbits, gsize) + plane_bytes(vbits); }
// metadata record group of 32-channel group g32: g32 >> meta_shift(G)
constexpr int meta_shift(int gsize) { return gsize == 32 ? 0 : (gsize == 64 ? 1 : 2); }

}  // namespace kvq
