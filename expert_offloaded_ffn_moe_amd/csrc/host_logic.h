// Host-side logic of the MoE offload library that needs no GPU: configuration
// checks, the internal expert layout and the canonical -> internal repack, and
// the expert-cache policy. Built into the library and, on its own with g++,
// into the CPU unit tests.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "moe_offload.h"

namespace moe {

// Internal expert layout (all regions 256-byte aligned inside one blob).
//
// Codes travel in 16-byte lane words: a word holds kc = 32 values of K for 4-bit
// codes and kc = 64 values for 2- and 3-bit codes (their low two bits; the third
// bit of 3-bit codes sits in a separate 8-byte "high plane" word per lane).
// Gate/up codes: tiles of 32 output positions; tile t, chunk c (kc values of K=H)
// is a 1 KiB block of 64 lanes x 16 bytes. Lane l < 32 holds gate row 32t+l,
// lane l >= 32 up row 32t+l-32, K range [kc*c, kc*c+kc).
// Down codes: tiles of 64 output rows; tile t, chunk c (kc values of K=I) is a
// 1 KiB block, lane l holds row 64t+l.
// Inside a 4-bit lane word, dword d covers K offsets [8d, 8d+8): the value at
// offset 8d+2j sits in bits [4j, 4j+4), at 8d+2j+1 in bits [16+4j, 20+4j),
// stored as n = q + 8 (0..15).
// Inside a 2- or 3-bit lane word, dword d covers K offsets [16d, 16d+16): the low
// two bits of code n at offset 16d+2j sit in bits [2j, 2j+2), at 16d+2j+1 in bits
// [16+2j, 18+2j). In the 3-bit high-plane word (same block order, 512 bytes per
// block), dword e covers offsets [32e, 32e+32): bit 2 of the code at 32e+2i is bit
// i, at 32e+2i+1 bit 16+i.
// Scales: per tile, one 128-byte row per quantisation group: lane l's fp16
// scale of that group for its row at bytes [2l, 2l+2).
struct Layout {
  int64_t H = 0, I = 0, G = 0, bits = 4, kc = 32;
  int64_t gu_tiles = 0, gu_chunks = 0, gu_groups = 0;
  int64_t dn_tiles = 0, dn_chunks = 0, dn_groups = 0;
  int64_t off_gu_codes = 0, off_gu_hi = 0, off_gu_scales = 0, off_dn_codes = 0, off_dn_hi = 0, off_dn_scales = 0;
  int64_t bytes = 0;            // internal blob size (multiple of 256)
  int64_t canonical_bytes = 0;  // 3*H*I*bits/8 + 6*H*I/G
};

Layout make_layout(int64_t H, int64_t I, int64_t G, int64_t bits = 4);

// Bits per weight code of cfg (weight_bits, 0 meaning 4).
inline int cfg_bits(const moe_config& c) { return c.weight_bits == 0 ? 4 : c.weight_bits; }

// Checks cfg; returns an empty string when valid, else the reason.
std::string check_config(const moe_config& c);

// canonical blob (layout documented in moe_offload.h) -> internal blob of L.bytes
void repack_expert(const Layout& L, const uint8_t* canonical, uint8_t* internal);

// One expert-cache update (frequency policy).
//   score[e] <- decay * score[e] + counts[e]
//   wanted: the first n_slots experts ordered by (score desc, resident first, id asc)
//   promotions: wanted non-residents ordered by (score desc, id asc), at most
//     max_promotions; each takes the lowest empty slot while one is left, else the
//     slot of the next victim, victims being residents not wanted, ordered by
//     (score asc, id desc).
// slot_of[e] is the HBM slot of e or -1. Updates score and slot_of in place.
struct Promotion {
  int32_t expert, slot;
};
void cache_policy_step(int32_t E, int32_t n_slots, double decay, int32_t max_promotions,
                       const int64_t* counts, double* score, int32_t* slot_of,
                       std::vector<Promotion>* promoted, std::vector<int32_t>* evicted);

// An update to a residency set the caller chose (want[e] != 0: read from HBM).
//   score[e] <- decay * score[e] + counts[e] (as in cache_policy_step)
//   evictions: residents not wanted, ascending id; their slots become free
//   promotions: wanted non-residents, ascending id, each into the lowest free slot
// Returns false (nothing changed) when more than n_slots experts are wanted.
bool cache_set_resident(int32_t E, int32_t n_slots, double decay, const int64_t* counts, const int32_t* want,
                        double* score, int32_t* slot_of, std::vector<Promotion>* promoted,
                        std::vector<int32_t>* evicted);

}  // namespace moe
