// SHA-256 (FIPS PUB 180-4, section 6.2), host only.
//
// The block manager keys a cached block by a chained digest of the whole token
// prefix that ends with it, so that two different prefixes can share a key
// only through a SHA-256 collision.  The round constants and the initial hash
// value are not typed in: they are derived at first use from their definition
// in FIPS 180-4 section 4.2.2 / 5.3.3 (the first 32 bits of the fractional
// parts of the cube roots of the first 64 primes, and of the square roots of
// the first 8 primes), with exact integer roots.
#pragma once

#include <cstddef>
#include <cstdint>
#include <cstring>

namespace pa {

struct Digest {
  uint8_t b[32];
  bool operator==(const Digest& o) const { return std::memcmp(b, o.b, 32) == 0; }
};

struct DigestHash {
  size_t operator()(const Digest& d) const {
    uint64_t h;
    std::memcpy(&h, d.b, 8);
    return static_cast<size_t>(h);
  }
};

namespace sha256_detail {

struct Tables {
  uint32_t k[64];
  uint32_t h0[8];
};

// largest x with x^e <= v (e = 2 or 3), by bisection on exact 128-bit integers
inline uint64_t iroot(unsigned __int128 v, int e, uint64_t hi) {
  uint64_t lo = 0;
  while (lo < hi) {
    const uint64_t mid = lo + (hi - lo + 1) / 2;
    unsigned __int128 p = mid;
    for (int i = 1; i < e; ++i) p *= mid;
    if (p <= v) lo = mid; else hi = mid - 1;
  }
  return lo;
}

inline Tables make_tables() {
  Tables t{};
  int found = 0;
  for (uint32_t n = 2; found < 64; ++n) {
    bool prime = true;
    for (uint32_t d = 2; d * d <= n; ++d)
      if (n % d == 0) { prime = false; break; }
    if (!prime) continue;
    // floor(cbrt(n) * 2^32) = floor(cbrt(n * 2^96)); keep its low 32 bits
    t.k[found] = static_cast<uint32_t>(iroot(static_cast<unsigned __int128>(n) << 96, 3, uint64_t(1) << 40));
    // floor(sqrt(n) * 2^32) = floor(sqrt(n * 2^64))
    if (found < 8)
      t.h0[found] = static_cast<uint32_t>(iroot(static_cast<unsigned __int128>(n) << 64, 2, uint64_t(1) << 40));
    ++found;
  }
  return t;
}

inline const Tables& tables() {
  static const Tables t = make_tables();
  return t;
}

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

inline void compress(uint32_t h[8], const uint8_t blk[64], const uint32_t k[64]) {
  uint32_t w[64];
  for (int i = 0; i < 16; ++i)
    w[i] = (uint32_t(blk[4 * i]) << 24) | (uint32_t(blk[4 * i + 1]) << 16) |
           (uint32_t(blk[4 * i + 2]) << 8) | uint32_t(blk[4 * i + 3]);
  for (int i = 16; i < 64; ++i) {
    const uint32_t s0 = rotr(w[i - 15], 7) ^ rotr(w[i - 15], 18) ^ (w[i - 15] >> 3);
    const uint32_t s1 = rotr(w[i - 2], 17) ^ rotr(w[i - 2], 19) ^ (w[i - 2] >> 10);
    w[i] = w[i - 16] + s0 + w[i - 7] + s1;
  }
  uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
  for (int i = 0; i < 64; ++i) {
    const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
    const uint32_t ch = (e & f) ^ (~e & g);
    const uint32_t t1 = hh + S1 + ch + k[i] + w[i];
    const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
    const uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
    const uint32_t t2 = S0 + maj;
    hh = g;
    g = f;
    f = e;
    e = d + t1;
    d = c;
    c = b;
    b = a;
    a = t1 + t2;
  }
  h[0] += a; h[1] += b; h[2] += c; h[3] += d;
  h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
}

}  // namespace sha256_detail

// Incremental SHA-256: update() with any number of byte strings, then
// finish() (padding per FIPS 180-4 section 5.1.1).  Allocates nothing.
class Sha256 {
 public:
  Sha256() { std::memcpy(h_, sha256_detail::tables().h0, sizeof h_); }

  void update(const uint8_t* data, size_t len) {
    const uint32_t* k = sha256_detail::tables().k;
    total_ += len;
    while (len > 0) {
      const size_t take = len < 64 - fill_ ? len : 64 - fill_;
      std::memcpy(buf_ + fill_, data, take);
      fill_ += take;
      data += take;
      len -= take;
      if (fill_ == 64) {
        sha256_detail::compress(h_, buf_, k);
        fill_ = 0;
      }
    }
  }

  Digest finish() {
    const uint64_t bits = total_ * 8;
    const uint8_t one = 0x80, zero = 0;
    update(&one, 1);
    while (fill_ != 56) update(&zero, 1);
    uint8_t len_be[8];
    for (int i = 0; i < 8; ++i) len_be[i] = static_cast<uint8_t>(bits >> (56 - 8 * i));
    update(len_be, 8);
    Digest d;
    for (int i = 0; i < 8; ++i) {
      d.b[4 * i] = static_cast<uint8_t>(h_[i] >> 24);
      d.b[4 * i + 1] = static_cast<uint8_t>(h_[i] >> 16);
      d.b[4 * i + 2] = static_cast<uint8_t>(h_[i] >> 8);
      d.b[4 * i + 3] = static_cast<uint8_t>(h_[i]);
    }
    return d;
  }

 private:
  uint32_t h_[8];
  uint8_t buf_[64];
  size_t fill_ = 0;
  uint64_t total_ = 0;
};

inline Digest sha256(const uint8_t* data, size_t len) {
  Sha256 h;
  h.update(data, len);
  return h.finish();
}

}  // namespace pa
