"""MI355X-native Clebsch-Gordan tensor-product (CGTP) convolution."""
