// Prints the library's SHA-256 of each command-line argument (as bytes) and of
// a few generated strings, one hex digest per line, for comparison with
// Python's hashlib in tests/test_host_sanitized.py.
#include <cstdio>
#include <cstring>
#include <string>

#include "sha256.hpp"

static void put(const std::string& s) {
  const pa::Digest d = pa::sha256(reinterpret_cast<const uint8_t*>(s.data()), s.size());
  for (int i = 0; i < 32; ++i) std::printf("%02x", d.b[i]);
  std::printf("\n");
}

int main(int argc, char** argv) {
  for (int i = 1; i < argc; ++i) put(argv[i]);
  // every length from 0 to 200 crosses the one- and two-block padding cases
  for (int n = 0; n <= 200; ++n) {
    std::string s;
    for (int i = 0; i < n; ++i) s.push_back(static_cast<char>((i * 7 + n) & 0xff));
    put(s);
  }
  return 0;
}
